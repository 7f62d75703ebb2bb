"""Bit-exact GPU parity for the layer's byte and index work, against the oracle.

* e4m3 activation quantisation ("Lab notes #6 ...", intro: w8a8 with per-token, per-128-column
  activation scales; "PR #39593 ...", Root cause: the fminf/fmaxf clamp to +-448): the codes and
  fp32 scales of every producer -- the quantisation kernel (fmoe_act_quant), the router launch
  that quantises x inside the forward, the separate pass over the gate/up activation, and the
  gate/up kernel's own epilogue -- equal oracle.act_quant on the same fp32 input, byte for byte,
  including all-zero groups, NaN, +-448, e4m3 rounding midpoints and their neighbours.
* Grouped GEMM indexing on integer data (every operand a small integer times a power-of-two
  scale, so every sum is exact in fp32): every kernel -- streaming light tiles, light tiles with
  the reduction split over 2 or 4 wavefronts, several light tiles per expert, heavy tiles of
  16..320 rows (320: one tile for an expert of 257..320 rows, bf16) -- gives outputs bit-equal to the oracle's, on every grouped row, with ragged and
  empty experts, repeated and out-of-range ids and an expert-parallel rank.
"""
import numpy as np
import pytest
import torch

import mixture_experts_layer_sigmoid_amd as fm
import oracle
from mixture_experts_layer_sigmoid_amd import synth
from gpu_common import Layer, announce

pytestmark = pytest.mark.gpu

E4M3_POS = np.array([oracle.e4m3_decode(c) for c in range(0x7F)], np.float64)  # 0x00..0x7E, ascending


def bf16_values(a: np.ndarray) -> np.ndarray:
    """float -> the bf16 value it rounds to (RNE), as fp32."""
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).float().numpy()


def special_groups(dtype) -> np.ndarray:
    """Rows of 128-column groups that reach the quantiser's edge cases; dtype 'bf16' keeps every
    value representable in bf16."""
    mids = (E4M3_POS[:-1] + E4M3_POS[1:]) / 2  # rounding midpoints below 448
    groups = []
    # amax = 448 exactly (scale 1, codes = e4m3(x)): midpoints, representable values, negatives
    for vals in (mids, E4M3_POS[1:], -mids):
        for i in range(0, len(vals), 127):
            g = np.zeros(128, np.float64)
            g[0] = 448.0
            chunk = vals[i:i + 127]
            g[1:1 + len(chunk)] = chunk
            groups.append(g)
    g = np.zeros(128)  # all zero: scale 1, codes 0
    groups.append(g)
    g = np.full(128, -0.0)  # negative zeros
    groups.append(g)
    g = np.linspace(-3, 3, 128)
    g[5] = np.nan  # NaN clamps to +448; amax ignores it
    groups.append(g)
    g = np.linspace(-1e30, 1e30, 128)  # huge values, scale far from 1
    groups.append(g)
    g = np.linspace(-1e-30, 1e-30, 128)  # tiny values: codes in the subnormal range
    groups.append(g)
    g = np.zeros(128)
    g[17] = -7.0  # one negative non-zero value: it becomes -448
    groups.append(g)
    x = np.stack(groups)
    if dtype == "bf16":
        x = bf16_values(x)
    return x.astype(np.float32)


def neighbours_of_midpoints() -> np.ndarray:
    """fp32 groups with 448 first, then each e4m3 midpoint's fp32 neighbours below and above."""
    mids = ((E4M3_POS[:-1] + E4M3_POS[1:]) / 2).astype(np.float32)
    vals = np.concatenate([np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(np.inf)), mids])
    vals = np.concatenate([vals, -vals])
    rows = []
    for i in range(0, len(vals), 127):
        g = np.zeros(128, np.float32)
        g[0] = 448.0
        chunk = vals[i:i + 127]
        g[1:1 + len(chunk)] = chunk
        rows.append(g)
    return np.stack(rows)


def compare_quant(q_gpu, s_gpu, x_f32, what):
    q_ref, s_ref = oracle.act_quant(x_f32)
    q_gpu = np.asarray(q_gpu)
    s_gpu = np.asarray(s_gpu)
    bad = np.argwhere(q_gpu != q_ref)
    assert bad.size == 0, f"{what}: {len(bad)} codes differ, first at {bad[0]}: gpu {q_gpu[tuple(bad[0])]:#04x} " \
                          f"oracle {q_ref[tuple(bad[0])]:#04x} for x={x_f32[tuple(bad[0])]!r}"
    assert np.array_equal(s_gpu.view(np.uint32), s_ref.view(np.uint32)), f"{what}: scales differ"
    # the largest magnitude of every group with a non-zero value encodes to +-448
    G = x_f32.shape[1] // 128
    for r in range(x_f32.shape[0]):
        for gi in range(G):
            grp = x_f32[r, gi * 128:(gi + 1) * 128]
            if np.isnan(grp).any() or not np.any(grp != 0):
                continue
            j = int(np.argmax(np.abs(grp)))
            assert q_gpu[r, gi * 128 + j] & 0x7F == 0x7E, f"{what}: amax of row {r} group {gi} is not +-448"


# ----------------------------------------------------------------------------- quantisation kernel

@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("rows,cols", [(1, 128), (7, 384), (301, 2048), (3, 7168)])
def test_quantisation_kernel_matches_oracle_bit_for_bit(dtype, rows, cols):
    announce(f"fmoe_act_quant {dtype} rows={rows} cols={cols}")
    g = np.random.default_rng(rows * 7 + cols)
    x = (g.standard_normal((rows, cols)) * np.exp(g.uniform(-8, 8, (rows, 1)))).astype(np.float32)
    if dtype == "bf16":
        x = bf16_values(x)
    sp = special_groups(dtype).reshape(-1)
    flat = x.reshape(-1)
    n = min(len(sp), len(flat))
    flat[:n] = sp[:n]  # as many of the special groups as fit
    xt = torch.from_numpy(x)
    xt = xt.to(torch.bfloat16) if dtype == "bf16" else xt
    q, s = fm.fmoe_act_quant(xt.cuda())
    torch.cuda.synchronize()
    compare_quant(q.cpu().numpy(), s.cpu().numpy(), x, f"quantisation kernel {dtype}")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_quantisation_kernel_special_groups(dtype):
    announce(f"fmoe_act_quant special groups {dtype}")
    x = special_groups(dtype)
    xt = torch.from_numpy(x)
    xt = xt.to(torch.bfloat16) if dtype == "bf16" else xt
    q, s = fm.fmoe_act_quant(xt.cuda())
    compare_quant(q.cpu().numpy(), s.cpu().numpy(), x, f"special groups {dtype}")
    r, c = np.argwhere(np.isnan(x))[0]
    assert q[r, c].item() == 0x7E  # NaN clamps to +448


def test_e4m3_conversion_at_midpoint_neighbours_and_random_values():
    """With 448 in the group the scale is 1, so the codes are the conversion of the values
    themselves: every midpoint, its fp32 neighbours, and 2^20 random values of every binade."""
    announce("e4m3 conversion: midpoints, neighbours, 2^20 random values")
    x1 = neighbours_of_midpoints()
    g = np.random.default_rng(5)
    mag = np.exp2(g.uniform(-12, np.log2(448.0), (8192, 127))).astype(np.float32)
    sgn = np.where(g.random((8192, 127)) < 0.5, -1.0, 1.0).astype(np.float32)
    x2 = np.concatenate([np.full((8192, 1), 448.0, np.float32), mag * sgn], 1)
    x = np.concatenate([x1, x2])
    q, s = fm.fmoe_act_quant(torch.from_numpy(x).cuda())
    assert torch.all(s == 1.0)
    compare_quant(q.cpu().numpy(), s.cpu().numpy(), x, "conversion")


# ----------------------------------------------------------------------------- quantisation inside the forward

def with_special_rows(L: Layer):
    """x of the layer with edge-case groups in its first rows (all-zero, NaN, +-448, midpoints)."""
    x = L.x.float().numpy().copy()
    sp = special_groups("bf16").reshape(-1)
    flat = x.reshape(-1)
    n = min(len(sp), len(flat) // 2)
    flat[:n] = sp[:n]
    L.x = torch.from_numpy(x).to(torch.bfloat16)
    L.x_gpu = L.x.cuda()


@pytest.mark.parametrize("T,H,I,E,k", [(12, 384, 256, 8, 2),      # fused router + grouping launch
                                       (40, 1024, 256, 16, 4),    # router kernel + quantising workgroups
                                       (288, 7168, 256, 400, 6)])  # the 7168-wide shard
def test_router_launch_x_codes_match_oracle(T, H, I, E, k):
    announce(f"x codes from the router launch T={T} H={H} E={E} k={k}")
    L = Layer(config=110, T=T, H=H, I=I, E=E, k=k, fp8=True, ep_size=8 if E == 400 else 1)
    with_special_rows(L)
    ws = fm.workspace(L.shape)
    L.forward(ws)
    torch.cuda.synchronize()
    lay = fm.fmoe_workspace_layout(L.shape)
    q = fm.ws_view(ws, lay["x_codes"], torch.uint8, (T, H)).cpu().numpy()
    s = fm.ws_view(ws, lay["x_scales"], torch.float32, (T, H // 128)).cpu().numpy()
    compare_quant(q, s, L.x.float().numpy(), "router-launch x")


@pytest.mark.parametrize("routing", ["uniform", "concentrated"])
def test_activation_quantisation_pass_matches_oracle(routing):
    """FP8 forward with heavy tiles possible: the gate/up kernels write the fp32 activation and
    a separate quantisation pass encodes it; its codes equal the oracle's on that fp32 input."""
    announce(f"h codes from the quantisation pass (heavy tiles possible), {routing}")
    L = Layer(config=synth.FP8_LAYER, weight_config=synth.BF16_LAYER, T=256, H=2048, I=768, E=128, k=8, fp8=True,
              routing=routing)
    L.plan = fm.fmoe_plan(32, 1, 1, 1)  # one light tile per expert: heavy launch, separate quantisation
    ws = fm.workspace(L.shape)
    L.forward(ws)
    st = fm.fmoe_read_stats(ws)
    R = st["local_rows"]
    lay = fm.fmoe_workspace_layout(L.shape)
    h = fm.ws_view(ws, lay["h_f32"], torch.float32, (R, 768)).cpu().numpy()
    q = fm.ws_view(ws, lay["h_codes"], torch.uint8, (R, 768)).cpu().numpy()
    s = fm.ws_view(ws, lay["h_scales"], torch.float32, (R, 6)).cpu().numpy()
    if routing == "concentrated":
        assert st["heavy_tiles"] > 0
    compare_quant(q, s, h, f"h quantisation pass ({routing})")


@pytest.mark.parametrize("T,H,I,E,k,tile", [(60, 512, 384, 8, 4, 32), (30, 256, 1024, 2, 2, 16)])
def test_gate_up_epilogue_codes_match_oracle(T, H, I, E, k, tile):
    """The gate/up kernel that quantises its own output (light tiles only, no split): codes equal
    the oracle's encoding of the fp32 activation the same tiles produce unquantised."""
    announce(f"h codes from the gate/up epilogue T={T} H={H} I={I} E={E} k={k} tile={tile}")
    L = Layer(config=111, T=T, H=H, I=I, E=E, k=k, fp8=True)
    ids = torch.from_numpy(np.random.default_rng(T).integers(0, E, (T, k)).astype(np.int32)).cuda()
    xq, xs = fm.fmoe_act_quant(L.x_gpu)
    plan = fm.fmoe_plan(tile, 1, 1, 8)
    h32 = fm.fmoe_grouped_gemm(L.shape, 0, ids, xq, L.w, a_scale=xs, out_dtype=fm.FMOE_FP32, plan=plan)
    ws = fm.workspace(L.shape)
    q, s = fm.fmoe_grouped_gemm(L.shape, 0, ids, xq, L.w, a_scale=xs, out_dtype=fm.FMOE_FP8_E4M3, plan=plan, ws=ws)
    st = fm.fmoe_read_stats(ws)
    assert st["heavy_tiles"] == 0 and st["max_rows"] > tile  # several light tiles for some expert
    R = st["local_rows"]
    compare_quant(q[:R].cpu().numpy(), s[:R].cpu().numpy(), h32[:R].cpu().numpy(), "gate/up epilogue")


# ----------------------------------------------------------------------------- integer-data grouped GEMMs

# rows per local expert: empty, single rows, both sides of every tile size, heavy tiles of
# 1..4 staged 64-row groups, experts cut into two and three heavy tiles; with one tile for
# 257..320 rows (bf16 plans with heavy_rows 320) 257 and 320 are tiles of five row groups
COUNTS = [0, 1, 15, 16, 17, 31, 32, 33, 64, 65, 128, 129, 256, 257, 320, 513]


def crafted_ids(counts, T, k, E, seed, lo=0):
    flat = np.concatenate([np.full(c, lo + e, np.int32) for e, c in enumerate(counts)])
    n = T * k
    assert len(flat) <= n
    pad = np.where(np.arange(n - len(flat)) % 2 == 0, -1, E + 5).astype(np.int32)  # dropped ids
    ids = np.concatenate([flat, pad])
    return np.random.default_rng(seed).permutation(ids).reshape(T, k)


E4M3_OF = {-2.0: 0xC0, -1.0: 0xB8, 0.0: 0x00, 1.0: 0x38, 2.0: 0x40}


def codes_of(v: np.ndarray) -> np.ndarray:
    out = np.zeros(v.shape, np.uint8)
    for val, c in E4M3_OF.items():
        out[v == val] = c
    return out


class IntCase:
    """Integer operands: gate/up stage a in {1,2}, gate weights in {1,2} (every gate sum is at
    least H, so silu(g) = g exactly on both sides), up and down weights and down-stage
    activations in {-2..2}; FP8 scales 1 or 2 (gate side) or 0.5..2 (up, down, activations)."""

    def __init__(self, T, k, E, H, I, fp8, counts, ep_size=1, ep_rank=0, seed=0):
        g = np.random.default_rng(seed)
        self.T, self.k, self.E, self.H, self.I, self.fp8 = T, k, E, H, I, fp8
        self.ep_size, self.ep_rank = ep_size, ep_rank
        El = E // ep_size
        lo = ep_rank * El
        # every expert gets its count; with EP the other ranks' experts take the rest of COUNTS
        full = list(counts) + [0] * (E - len(counts))
        self.ids = crafted_ids(full[:E], T, k, E, seed)
        self.shape = fm.make_shape(T, H, I, E, k, ep_size, ep_rank, fp8)
        self.x = g.integers(1, 3, (T, H)).astype(np.float32)
        self.wg = g.integers(1, 3, (El, I, H)).astype(np.float32)
        self.wu = g.integers(-2, 3, (El, I, H)).astype(np.float32)
        self.wd = g.integers(-2, 3, (El, H, I)).astype(np.float32)
        self.h = g.integers(-2, 3, (T * k, I)).astype(np.float32)
        if fp8:
            pick = lambda vals, shape: np.asarray(vals, np.float32)[g.integers(0, len(vals), shape)]
            self.xs = pick([1.0, 2.0], (T, H // 128))
            self.hs = pick([0.5, 1.0, 2.0], (T * k, I // 128))
            self.sg = pick([1.0, 2.0], (El, I // 128, H // 128))
            self.su = pick([0.5, 1.0, 2.0], (El, I // 128, H // 128))
            self.sd = pick([0.5, 1.0, 2.0], (El, H // 128, I // 128))
            cu = lambda a: torch.from_numpy(codes_of(a)).cuda()
            self.w = fm.ExpertWeights(cu(self.wg), cu(self.wu), cu(self.wd), torch.from_numpy(self.sg).cuda(),
                                      torch.from_numpy(self.su).cuda(), torch.from_numpy(self.sd).cuda())
        else:
            bf = lambda a: torch.from_numpy(a).to(torch.bfloat16).cuda()
            self.w = fm.ExpertWeights(bf(self.wg), bf(self.wu), bf(self.wd))
        self.R = int(oracle.route_permute(self.ids, E, ep_size, ep_rank)["offsets"][-1])

    def bits(self, a):
        return synth.bf16_bits(torch.from_numpy(a).to(torch.bfloat16))

    def oracle_stage(self, stage):
        kw = dict(ep_size=self.ep_size, ep_rank=self.ep_rank)
        if self.fp8:
            if stage == 0:
                return oracle.grouped_gemm(0, self.ids, self.E, codes_of(self.x), codes_of(self.wg), codes_of(self.wu),
                                           a_scale=self.xs, s0=self.sg, s1=self.su, **kw)
            return oracle.grouped_gemm(1, self.ids, self.E, codes_of(self.h), codes_of(self.wd), a_scale=self.hs,
                                       s0=self.sd, **kw)
        if stage == 0:
            return oracle.grouped_gemm(0, self.ids, self.E, self.bits(self.x), self.bits(self.wg), self.bits(self.wu),
                                       **kw)
        return oracle.grouped_gemm(1, self.ids, self.E, self.bits(self.h), self.bits(self.wd), **kw)

    def gpu_stage(self, stage, plan, out_dtype=None, ws=None):
        ids = torch.from_numpy(self.ids).cuda()
        if self.fp8:
            a = torch.from_numpy(codes_of(self.x if stage == 0 else self.h)).cuda()
            sc = torch.from_numpy(self.xs if stage == 0 else self.hs).cuda()
        else:
            a = torch.from_numpy(self.x if stage == 0 else self.h).to(torch.bfloat16).cuda()
            sc = None
        return fm.fmoe_grouped_gemm(self.shape, stage, ids, a, self.w, a_scale=sc, out_dtype=out_dtype, plan=plan,
                                    ws=ws)


def assert_bits_equal(got: torch.Tensor, ref_f64: np.ndarray, what: str):
    """GPU output (bf16 or fp32) against the exact oracle value rounded once to that format."""
    ref32 = torch.from_numpy(ref_f64.astype(np.float32))
    ref = ref32.to(got.dtype)
    g = got.cpu()
    eq = g.view(torch.int16 if got.dtype == torch.bfloat16 else torch.int32) == \
        ref.view(torch.int16 if got.dtype == torch.bfloat16 else torch.int32)
    if not bool(eq.all()):
        r, c = (~eq).nonzero()[0].tolist()
        raise AssertionError(f"{what}: {int((~eq).sum())} values differ, first at row {r} col {c}: "
                             f"gpu {g[r, c].item()} oracle {ref_f64[r, c]}")


PLANS = {  # (tile rows, gate/up split, down split, light tiles per expert, heavy rows: 320 for bf16)
    "stream16": (16, 1, 1, 1, 320), "stream32": (32, 1, 1, 1, 256),
    "split2_16": (16, 2, 2, 1, 256), "split4_32": (32, 4, 4, 1, 320),
}


def plan_for(name: str, fp8: bool):
    tr, s1, s2, lt, hr = PLANS[name]
    return fm.fmoe_plan(tr, s1, s2, lt, 0 if fp8 else hr)


@pytest.mark.parametrize("H,I", [(256, 384), (640, 256), (1152, 896), (512, 768)])
@pytest.mark.parametrize("plan", list(PLANS))
@pytest.mark.parametrize("fp8", [False, True])
def test_integer_grouped_gemm_is_bit_exact(fp8, plan, H, I):
    announce(f"integer grouped GEMM fp8={fp8} plan={plan} H={H} I={I}")
    C = IntCase(T=470, k=4, E=16, H=H, I=I, fp8=fp8, counts=COUNTS, seed=H + I)
    p = plan_for(plan, fp8)
    ws = fm.workspace(C.shape)
    out0 = C.gpu_stage(0, p, ws=ws)
    st = fm.fmoe_read_stats(ws)
    assert st["local_rows"] == C.R == sum(COUNTS) and st["dropped_ids"] == C.T * C.k - sum(COUNTS)
    five = not fp8 and PLANS[plan][4] == 320
    heavy = [c for c in COUNTS if c > PLANS[plan][0]]
    assert st["heavy_rows"] == (320 if five else 256)
    assert st["heavy_tiles"] == sum(1 if five and 256 < c <= 320 else -(-c // 256) for c in heavy)
    torch.cuda.synchronize()
    ref0 = C.oracle_stage(0)
    assert_bits_equal(out0[:C.R], ref0, "gate/up")
    if fp8:  # the same stage with e4m3 output: separate quantisation pass over the fp32 activation
        q, s = C.gpu_stage(0, p, out_dtype=fm.FMOE_FP8_E4M3)
        compare_quant(q[:C.R].cpu().numpy(), s[:C.R].cpu().numpy(), ref0.astype(np.float32), "gate/up codes")
    out1 = C.gpu_stage(1, p)
    assert_bits_equal(out1[:C.R], C.oracle_stage(1), "down")


@pytest.mark.parametrize("fp8", [False, True])
def test_integer_grouped_gemm_expert_parallel_rank(fp8):
    announce(f"integer grouped GEMM, rank 1 of 2, fp8={fp8}")
    C = IntCase(T=470, k=4, E=16, H=384, I=256, fp8=fp8, counts=COUNTS, ep_size=2, ep_rank=1, seed=3)
    for plan in ("stream16", "split2_16"):
        p = plan_for(plan, fp8)
        assert C.R == sum(COUNTS[8:])
        assert_bits_equal(C.gpu_stage(0, p)[:C.R], C.oracle_stage(0), f"gate/up {plan}")
        assert_bits_equal(C.gpu_stage(1, p)[:C.R], C.oracle_stage(1), f"down {plan}")


@pytest.mark.parametrize("split", [1, 2, 4])
@pytest.mark.parametrize("fp8", [False, True])
def test_integer_grouped_gemm_several_light_tiles_per_expert(fp8, split):
    """Every expert fits 8 light tiles of 32 rows (240 assignments), so no heavy launch: experts
    of 33..96 rows are cut into several light tiles; FP8 gate/up without a split writes its codes
    itself."""
    announce(f"integer grouped GEMM, light tiles only, fp8={fp8} split={split}")
    counts = [0, 1, 31, 32, 33, 64, 79]
    C = IntCase(T=60, k=4, E=8, H=512, I=384, fp8=fp8, counts=counts, seed=11 + split)
    p = fm.fmoe_plan(32, split, split, 8)
    ws = fm.workspace(C.shape)
    out0 = C.gpu_stage(0, p, ws=ws)
    st = fm.fmoe_read_stats(ws)
    assert st["heavy_tiles"] == 0 and st["m_tiles"] == sum(-(-c // 32) for c in counts)
    ref0 = C.oracle_stage(0)
    assert_bits_equal(out0[:C.R], ref0, "gate/up")
    if fp8:
        q, s = C.gpu_stage(0, p, out_dtype=fm.FMOE_FP8_E4M3)
        compare_quant(q[:C.R].cpu().numpy(), s[:C.R].cpu().numpy(), ref0.astype(np.float32), "gate/up codes")
    assert_bits_equal(C.gpu_stage(1, p)[:C.R], C.oracle_stage(1), "down")
