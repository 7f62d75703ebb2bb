"""GPU parity of the whole layer against the oracle: routing bit-exact, outputs within
2e-2 (bf16) / 6e-2 (FP8) max row relative error; every token at the full workload sizes (so every
row tile and every 16-row block of a heavy tile is checked); edge cases."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_sigmoid_amd as fm
import oracle
from mixture_experts_layer_sigmoid_amd import synth
from gpu_common import BF16_TOL, FP8_TOL, Layer, announce, check_layer, row_rel_err, sample_tokens

ALL = 10 ** 9  # every token of the batch against the oracle (all row tiles and 16-row blocks)

pytestmark = pytest.mark.gpu


def test_tiny_layer_end_to_end():
    announce("tiny layer T=16 H=256 E=8 I=128 k=2")
    T, H, E, I, k = 16, 256, 8, 128, 2
    L = synth.tiny_layer(T, H, E, I)
    g = {n: t.cuda() for n, t in L.items()}
    logits = fm.fmoe_router_logits(g["x"], g["wr"])
    out, ids, wts = fm.fmoe_forward(fm.make_shape(T, H, I, E, k), g["x"], logits,
                                    fm.ExpertWeights(g["wg"], g["wu"], g["wd"]), return_routing=True)
    lg_ref = oracle.router_logits(synth.bf16_bits(L["x"]), synth.bf16_bits(L["wr"]))
    ids_ref, w_ref = oracle.router_topk(lg_ref, k, "softmax", True)
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    assert np.abs(wts.cpu().numpy() - w_ref).max() <= 1e-6
    ref = oracle.moe_tokens(synth.bf16_bits(L["x"]), ids_ref, w_ref,
                            *(synth.bf16_bits(L[n]) for n in ("wg", "wu", "wd")), E=E)
    assert row_rel_err(out.float().cpu().numpy(), ref) <= BF16_TOL


@pytest.mark.parametrize("T,H,I,E,k,routing,scoring", [
    (37, 512, 384, 16, 4, "uniform", "softmax"),      # several 16-row tiles and n-blocks, ragged
    (300, 256, 256, 8, 4, "uniform", "softmax"),      # estimate 150 -> 128-row tiles, 2 per expert
    (300, 256, 256, 8, 4, "concentrated", "sigmoid"),
    (130, 384, 128, 32, 8, "uniform", "sigmoid"),     # estimate 33 -> 64-row tiles
    (1, 256, 128, 8, 8, "uniform", "softmax"),        # k = E
])
def test_bf16_layer_small(T, H, I, E, k, routing, scoring):
    announce(f"bf16 layer T={T} H={H} I={I} E={E} k={k} {routing} {scoring}")
    L = Layer(config=90, T=T, H=H, I=I, E=E, k=k, routing=routing, scoring=scoring)
    check_layer(L, n_sample=10 ** 6)


@pytest.mark.parametrize("T,H,I,E,k,ep", [(50, 512, 256, 8, 2, 1), (40, 256, 384, 16, 6, 2), (200, 256, 256, 4, 2, 1),
                                          (20, 128, 128, 4, 2, 1),  # one 128-deep block: idle split-K waves
                                          (120, 256, 256, 8, 2, 1)])  # experts in 1-2 light tiles, no heavy tiles
def test_fp8_layer_small(T, H, I, E, k, ep):
    announce(f"fp8 layer T={T} H={H} I={I} E={E} k={k} ep={ep}")
    L = Layer(config=91, T=T, H=H, I=I, E=E, k=k, fp8=True, ep_size=ep, ep_rank=ep - 1)
    check_layer(L, n_sample=10 ** 6)


# The streaming light kernel (no split reduction, forced by the tile plan) on shapes covering
# 16- and 32-row tiles, single-chunk reductions, chunks padded past the reduction end (bf16
# chunks of 8 steps, FP8 of 4 or 6) and an expert-parallel shard.
@pytest.mark.parametrize("T,H,I,E,k,ep,fp8", [
    (64, 256, 512, 64, 8, 1, False),    # GEMM1 streamed, one chunk, 32-row tiles
    (40, 1024, 384, 64, 4, 1, False),   # GEMM2 streamed, 12 steps in 2 chunks, 16-row tiles
    (128, 1024, 1024, 64, 8, 1, True),  # FP8, both streamed
    (64, 384, 640, 64, 8, 1, True),     # FP8 GEMM1 with 3 steps in a 4-step chunk
    (96, 640, 256, 128, 8, 2, True),    # FP8 GEMM2 with 2 steps in a chunk, rank 1 of 2
])
def test_layer_streaming_kernel_shapes(T, H, I, E, k, ep, fp8):
    announce(f"streaming-kernel shape T={T} H={H} I={I} E={E} k={k} ep={ep} fp8={fp8}")
    L = Layer(config=94, T=T, H=H, I=I, E=E, k=k, fp8=fp8, ep_size=ep, ep_rank=ep - 1)
    L.plan = fm.fmoe_plan(0, 1, 1)
    check_layer(L, n_sample=10 ** 6)


# Experts cut into several light tiles (up to 8 per expert, the heavy-tile launches left out):
# hot experts of a concentrated routing span two or more 32-row tiles (at most T=120 rows),
# ragged last tiles; FP8 also quantises the activation in the gate/up kernel.
@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("routing", ["uniform", "concentrated"])
def test_layer_multi_light_tiles(fp8, routing):
    announce(f"several light tiles per expert, fp8={fp8} {routing}")
    L = Layer(config=95, T=120, H=256, I=384, E=16, k=4, fp8=fp8, routing=routing)
    L.plan = fm.fmoe_plan(32, 1, 1, 8)
    check_layer(L, n_sample=10 ** 6)
    ws = fm.workspace(L.shape)
    L.forward(ws)
    st = fm.fmoe_read_stats(ws)
    assert st["heavy_tiles"] == 0 and st["m_tiles"] >= -(-st["max_rows"] // 32)
    if routing == "concentrated":
        assert st["max_rows"] > 32  # hot experts take two light tiles or more


@pytest.mark.parametrize("T", [1, 8, 32, 128, 256, 512, 1024, 4096])
def test_bf16_layer_2048x768_e128_top8_uniform(T):
    announce(f"bf16 H=2048 I=768 E=128 k=8 uniform T={T}")
    L = Layer(config=synth.BF16_LAYER, T=T, H=2048, I=768, E=128, k=8)
    r = check_layer(L, n_sample=ALL)
    print(f"T={T} max row rel err {r['err']:.3e}")


@pytest.mark.parametrize("T", [32, 256, 4096])
def test_bf16_layer_2048x768_e128_top8_concentrated(T):
    announce(f"bf16 H=2048 I=768 E=128 k=8 concentrated T={T}")
    L = Layer(config=synth.BF16_LAYER, T=T, H=2048, I=768, E=128, k=8, routing="concentrated")
    check_layer(L, n_sample=ALL)


@pytest.mark.parametrize("routing", ["uniform", "concentrated"])
def test_light_gate_up_kernel_chosen_from_the_real_counts(routing):
    # T=256 of the 128-expert bf16 layer expects 16 rows per expert.  Uniform light tiles hold
    # about that many and stay on the streaming kernel; the cold experts of a concentrated batch
    # hold one or two rows each and the grouping hands them to the split-reduction kernel (the
    # hot experts are heavy tiles).  Either way the output equals, bit for bit, the forced plan
    # that runs the same kernel on the same tiles, and the oracle on every token.
    announce(f"bf16 T=256 {routing}: light gate/up kernel picked on the device")
    L = Layer(config=synth.BF16_LAYER, T=256, H=2048, I=768, E=128, k=8, routing=routing)
    ws = fm.workspace(L.shape)
    auto = L.forward(ws)[0].clone()
    st = fm.fmoe_read_stats(ws)
    light = st["m_tiles"] - st["heavy_tiles"]
    assert light > 0
    if routing == "concentrated":
        assert st["heavy_tiles"] > 0 and st["split_light_tiles"] == light and st["light_rows"] < 4 * light
        forced = fm.fmoe_plan(32, 2, 1, 1)  # the split-reduction gate/up kernel (two wavefronts)
    else:
        assert st["split_light_tiles"] == 0 and st["light_rows"] >= 4 * light
        forced = fm.fmoe_plan(32, 1, 1, 1)  # the streaming gate/up kernel
    L.plan = forced
    again = L.forward(ws)[0]
    assert fm.fmoe_read_stats(ws)["split_light_tiles"] == 0  # a forced split leaves the choice out
    assert torch.equal(again, auto)
    L.plan = None
    check_layer(L, n_sample=ALL)


@pytest.mark.parametrize("T", [128, 256])
def test_fp8_layer_2048x768_e128_top8_concentrated(T):
    # hot experts of ~120 / ~240 rows cut into 4 / 8 light tiles, no heavy launch
    announce(f"fp8 H=2048 I=768 E=128 k=8 concentrated T={T}")
    L = Layer(config=synth.FP8_LAYER, weight_config=synth.BF16_LAYER, T=T, H=2048, I=768, E=128, k=8, fp8=True,
              routing="concentrated")
    check_layer(L, n_sample=ALL)
    ws = fm.workspace(L.shape)
    L.forward(ws)
    st = fm.fmoe_read_stats(ws)
    assert st["heavy_tiles"] == 0 and st["max_rows"] > 2 * st["tile_rows"]


@pytest.mark.parametrize("T", [64, 128, 256])
def test_fp8_layer_2048x768_e128_top8(T):
    announce(f"fp8 H=2048 I=768 E=128 k=8 T={T}")
    L8 = Layer(config=synth.FP8_LAYER, weight_config=synth.BF16_LAYER, T=T, H=2048, I=768, E=128, k=8, fp8=True)
    check_layer(L8, n_sample=ALL)
    # beside the bf16 layer the weights were quantised from (information; loose bound)
    Lb = Layer(config=synth.FP8_LAYER, weight_config=synth.BF16_LAYER, T=T, H=2048, I=768, E=128, k=8)
    o8 = L8.forward()[0].float().cpu().numpy()
    ob = Lb.forward()[0].float().cpu().numpy()
    rel = row_rel_err(o8, ob)
    print(f"T={T} fp8 vs bf16 path max row rel diff {rel:.3e}")
    assert rel < 0.25


@pytest.mark.parametrize("routing", ["uniform", "concentrated"])
def test_fp8_local_shard_288_tokens_top6_of_400(routing):
    announce(f"fp8 H=7168 I=2048 E=400 (ep 8, rank 0) k=6 T=288 {routing}")
    L = Layer(config=synth.EP_SHARD, T=288, H=7168, I=2048, E=400, k=6, ep_size=8, ep_rank=0, fp8=True,
              routing=routing)
    check_layer(L, n_sample=ALL)


def test_experts_all_tokens_one_expert_duplicates_and_dropped_ids():
    announce("experts: all ids 0 (duplicates), out-of-range ids")
    T, H, I, E, k = 64, 256, 128, 8, 4
    L = synth.tiny_layer(T, H, E, I, seed=5)
    w = fm.ExpertWeights(L["wg"].cuda(), L["wu"].cuda(), L["wd"].cuda())
    shape = fm.make_shape(T, H, I, E, k)
    wts = np.random.default_rng(1).random((T, k)).astype(np.float32)
    bits = [synth.bf16_bits(L[n]) for n in ("wg", "wu", "wd")]
    for ids in (np.zeros((T, k), np.int32), np.random.default_rng(2).integers(-3, E + 3, (T, k)).astype(np.int32)):
        ws = fm.workspace(shape)
        out = fm.fmoe_experts(shape, L["x"].cuda(), torch.from_numpy(ids).cuda(), torch.from_numpy(wts).cuda(), w, ws=ws)
        ref = oracle.moe_tokens(synth.bf16_bits(L["x"]), ids, wts.astype(np.float64), *bits, E=E)
        assert row_rel_err(out.float().cpu().numpy(), ref) <= BF16_TOL
        st = fm.fmoe_read_stats(ws)
        assert st["dropped_ids"] == int(((ids < 0) | (ids >= E)).sum())


# The forward quantises x inside its router launch (the fused router + grouping launch up to 16
# tokens, the router kernel above); fmoe_experts runs the separate quantisation kernel.  Same
# codes and the same tile plan give the same output bits.
@pytest.mark.parametrize("T", [12, 100])
def test_fp8_forward_quantises_x_in_the_router_launch(T):
    announce(f"fp8 forward (x quantised by the router launch) == experts (quantisation kernel), T={T}")
    L = Layer(config=96, T=T, H=384, I=256, E=8, k=2, fp8=True)
    out, ids, wts = L.forward()
    out2 = fm.fmoe_experts(L.shape, L.x_gpu, ids, wts, L.w)
    assert torch.equal(out, out2)
    check_layer(L, n_sample=10 ** 6)


# The gate/up kernel that quantises h in its epilogue (light tiles only) against the separate
# quantisation kernel (used whenever heavy tiles may exist): on a batch whose experts all fit a
# light tile, both plans cut the same tiles, so the outputs must agree bit for bit.
@pytest.mark.parametrize("T,H,I,E,k", [(40, 256, 384, 16, 1), (60, 512, 256, 8, 2)])
def test_fp8_fused_h_quantisation_equals_the_quantisation_kernel(T, H, I, E, k):
    announce(f"fp8 fused h quantisation vs quantisation kernel T={T} H={H} I={I} E={E} k={k}")
    L = Layer(config=99, T=T, H=H, I=I, E=E, k=k, fp8=True)
    ws = fm.workspace(L.shape)
    L.plan = fm.fmoe_plan(32, 1, 1, 8)  # every expert light: gate/up writes e4m3 codes itself
    fused = L.forward(ws)[0]
    st = fm.fmoe_read_stats(ws)
    assert st["heavy_tiles"] == 0 and st["max_rows"] <= 32
    L.plan = fm.fmoe_plan(32, 1, 1, 1)  # heavy launch possible (T > 32): fp32 h, then the kernel
    separate = L.forward(ws)[0]
    assert fm.fmoe_read_stats(ws)["heavy_tiles"] == 0
    assert torch.equal(fused, separate)
    check_layer(L, n_sample=10 ** 6)


@pytest.mark.parametrize("T", [12, 40])
def test_fp8_nan_activation_rows_stay_in_their_tokens(T):
    announce(f"fp8 layer with NaN rows of x, T={T}")
    L = Layer(config=97, T=T, H=256, I=256, E=8, k=2, fp8=True)
    bad = [1, T - 2]
    x = L.x.clone()
    x[bad] = float("nan")
    L.x, L.x_gpu = x, x.cuda()
    out, ids, _ = L.forward()
    ids_ref, w_ref = L.oracle_routing()
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    others = np.array([t for t in range(T) if t not in bad], np.int32)
    got = out.float().cpu().numpy()
    assert np.isfinite(got).all()  # the quantiser clamps NaN to +448 (a finite code)
    ref = L.oracle_tokens(ids_ref, w_ref, others)
    assert row_rel_err(got[others], ref) <= FP8_TOL


def test_nan_logit_rows_give_distinct_experts_and_finite_output():
    announce("layer with all-NaN logit rows (padding tokens)")
    L = Layer(config=92, T=40, H=256, I=256, E=16, k=4)
    lg = L.logits.clone()
    lg[[3, 17, 39]] = float("nan")
    L.logits, L.logits_gpu = lg, lg.cuda()
    out, ids, _ = L.forward()
    ids = ids.cpu().numpy()
    for r in (3, 17, 39):
        assert ids[r].tolist() == [0, 1, 2, 3]
    assert torch.isfinite(out.float()).all()
    check_layer(L, n_sample=10 ** 6)


def test_empty_rank_tokens_are_zero():
    announce("expert-parallel rank with tokens routed elsewhere")
    L = Layer(config=93, T=64, H=256, I=128, E=32, k=2, ep_size=8, ep_rank=7)
    out, ids, _ = L.forward()
    ids = ids.cpu().numpy()
    none_local = ~np.any((ids >= 28) & (ids < 32), axis=1)
    assert none_local.any()
    assert torch.all(out[torch.from_numpy(none_local).cuda()] == 0)
    check_layer(L, n_sample=10 ** 6)


# Seeded random small shapes (T <= 64, E <= 16, k <= E, several H and I, bf16 and FP8, uniform and
# concentrated routing, softmax and sigmoid, expert-parallel ranks): routing bit-exact and
# outputs within the bars on every token.
@pytest.mark.parametrize("case", range(16))
def test_random_small_shapes_match_the_oracle(case):
    g = np.random.default_rng(1000 + case)
    E = int(g.choice([1, 2, 3, 4, 6, 8, 12, 16]))
    k = int(g.integers(1, E + 1))
    T = int(g.integers(1, 65))
    H = int(g.choice([128, 256, 384, 512]))
    I = int(g.choice([128, 256, 384]))
    ep = int(g.choice([d for d in (1, 2, 4) if E % d == 0]))
    rank = int(g.integers(0, ep))
    fp8 = bool(case % 2)
    routing = "concentrated" if case % 4 >= 2 and E > k else "uniform"  # concentration needs a cold expert
    scoring = "sigmoid" if case % 3 == 0 else "softmax"
    announce(f"random shape {case}: T={T} H={H} I={I} E={E} k={k} ep={ep}/{rank} fp8={fp8} {routing} {scoring}")
    L = Layer(config=200 + case, T=T, H=H, I=I, E=E, k=k, fp8=fp8, ep_size=ep, ep_rank=rank, routing=routing,
              scoring=scoring)
    check_layer(L, n_sample=10 ** 6)


# Heavy row tiles at the shortest reductions and at stage counts that end inside a cycle of the
# heavy kernel's buffer rings (bf16: 64-deep stages, 12 per cycle, 4 for tiles of five 64-row
# groups; FP8: 128-deep stages, 3 per cycle): K = 128 gives 2 bf16 stages and a single FP8 stage.
# About 300 rows per expert, so experts are cut into one or two heavy tiles (bf16 with one tile
# for 257..320 rows forced: tiles of five row groups).
@pytest.mark.parametrize("H,I", [(128, 128), (128, 384), (640, 256), (1152, 896)])
@pytest.mark.parametrize("fp8", [False, True])
def test_heavy_tiles_at_short_and_ragged_reductions(H, I, fp8):
    announce(f"heavy tiles H={H} I={I} fp8={fp8}")
    L = Layer(config=96, T=600, H=H, I=I, E=4, k=2, fp8=fp8)
    if not fp8:
        L.plan = fm.fmoe_plan(0, 0, 0, 0, 320)
    ws = fm.workspace(L.shape)
    L.forward(ws=ws)
    st = fm.fmoe_read_stats(ws)
    assert st["heavy_tiles"] >= 4 and st["heavy_rows"] == (256 if fp8 else 320)
    check_layer(L, n_sample=10 ** 6)


# The library's declared size limits and large batches: hidden or inter at 65536 (bf16 and FP8;
# FP8 32-row split tiles would overflow 64 KB of scales, so the plan takes 16-row tiles), 1024
# local experts with top-64 routing, one expert holding 65536 rows (256 heavy tiles), and 2^20
# assignments (16384 grouping chunks); sampled tokens against the oracle.
@pytest.mark.parametrize("T,H,I,E,k,fp8,n_sample", [
    (3, 65536, 128, 2, 2, False, 10 ** 6),
    (3, 65536, 128, 2, 1, True, 10 ** 6),
    (2, 128, 65536, 2, 1, False, 10 ** 6),
    (2, 128, 65536, 2, 2, True, 10 ** 6),
    (32, 128, 128, 1024, 64, False, 10 ** 6),
    (65536, 128, 128, 1, 1, False, 48),
    (131072, 128, 128, 16, 8, False, 48),
])
def test_size_limits_and_large_batches(T, H, I, E, k, fp8, n_sample):
    announce(f"size limits T={T} H={H} I={I} E={E} k={k} fp8={fp8}")
    L = Layer(config=97, T=T, H=H, I=I, E=E, k=k, fp8=fp8)
    check_layer(L, n_sample=n_sample)


@pytest.mark.parametrize("fp8", [False, True])
def test_all_assignments_on_one_expert_at_the_assignment_limit(fp8):
    # caller ids may repeat: 2^20 tokens x top-8, every id 0, is 2^23 rows (the limit) on one
    # expert, cut into 32768 heavy tiles (the count fills the top 16 bits of the tile field)
    T, H, I, E, k = 1 << 20, 128, 128, 8, 8
    announce(f"fmoe_experts: {T * k} rows on one expert, fp8={fp8}")
    x = synth.activations(98, T, H)
    ids = np.zeros((T, k), np.int32)
    wts = np.random.default_rng(3).random((T, k)).astype(np.float32)
    shape = fm.make_shape(T, H, I, E, k, fp8=fp8)
    ws = fm.workspace(shape)
    tok = sample_tokens(T, 48)
    if fp8:
        q = synth.expert_weights_fp8(4, E, H, I, 0, 7)
        w = fm.ExpertWeights(*(t.cuda() for t in q))
        qg, qu, qd, sg, su, sd = (t.numpy() for t in q)
        ref = oracle.moe_tokens(synth.bf16_bits(x), ids, wts.astype(np.float64), qg, qu, qd, E=E, sg=sg, su=su,
                                sd=sd, tokens=tok)
    else:
        L = synth.tiny_layer(4, H, E, I, seed=7)  # weights only
        w = fm.ExpertWeights(L["wg"].cuda(), L["wu"].cuda(), L["wd"].cuda())
        ref = oracle.moe_tokens(synth.bf16_bits(x), ids, wts.astype(np.float64),
                                *(synth.bf16_bits(L[n]) for n in ("wg", "wu", "wd")), E=E, tokens=tok)
    out = fm.fmoe_experts(shape, x.cuda(), torch.from_numpy(ids).cuda(), torch.from_numpy(wts).cuda(), w, ws=ws)
    st = fm.fmoe_read_stats(ws)
    assert st["local_rows"] == T * k and st["max_rows"] == T * k and st["heavy_tiles"] == T * k // 256
    assert st["heavy_rows"] == (256 if fp8 else 320)  # bf16: one tile for 257..320 rows (none here)
    assert row_rel_err(out.float().cpu().numpy()[tok], ref) <= (FP8_TOL if fp8 else BF16_TOL)
    del ws, out


def test_forward_is_deterministic_and_matches_experts():
    announce("determinism and forward == router + experts")
    L = Layer(config=synth.BF16_LAYER, T=256, H=2048, I=768, E=128, k=8, routing="concentrated")
    ws = fm.workspace(L.shape)
    first, ids, wts = L.forward(ws)
    for _ in range(100):
        again = L.forward(ws)[0]
        assert torch.equal(again, first)
    out2 = fm.fmoe_experts(L.shape, L.x_gpu, ids, wts, L.w)
    assert torch.equal(out2, first)


@pytest.mark.parametrize("fp8", [False, True])
def test_profiled_forward_and_hip_graph_replays_match_eager(fp8):
    """Eager, profiled (every stage event, or only the light gate/up pair) and graph-replayed
    calls with heavy row tiles are bitwise equal."""
    announce(f"profiled forward and HIP graph capture/replays vs eager (concentrated, heavy tiles, fp8={fp8})")
    L = Layer(config=synth.BF16_LAYER, T=512, H=2048, I=768, E=128, k=8, fp8=fp8, routing="concentrated")
    ws = fm.workspace(L.shape)
    eager = fm.fmoe_forward(L.shape, L.x_gpu, L.logits_gpu, L.w, ws=ws)
    assert fm.fmoe_read_stats(ws)["heavy_tiles"] > 0
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(fm.FMOE_NUM_STAGES + 1)]
    profiled = fm.fmoe_forward(L.shape, L.x_gpu, L.logits_gpu, L.w, ws=ws, stage_events=evs)
    assert torch.equal(profiled, eager)
    # only the event pair around the streaming gate/up GEMM (how the benchmark times it)
    pair = [None] * (fm.FMOE_NUM_STAGES + 1)
    pair[fm.STAGES.index("gemm1")] = torch.cuda.Event(enable_timing=True)
    pair[fm.STAGES.index("gemm1_split")] = torch.cuda.Event(enable_timing=True)
    assert torch.equal(fm.fmoe_forward(L.shape, L.x_gpu, L.logits_gpu, L.w, ws=ws, stage_events=pair), eager)
    out = torch.empty_like(eager)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fm.fmoe_forward(L.shape, L.x_gpu, L.logits_gpu, L.w, ws=ws, out=out)
    for i in range(3):
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i}"
        # eager work between the replays
        assert torch.equal(fm.fmoe_forward(L.shape, L.x_gpu, L.logits_gpu, L.w, ws=ws), eager)


@pytest.mark.parametrize("fp8", [False, True])
def test_every_tile_plan_matches_the_oracle(fp8):
    announce(f"all 36 tile plans (tile rows x gate/up split x down split x light tiles), concentrated, fp8={fp8}")
    T, H, I, E, k = 130, 384, 256, 32, 8
    L = Layer(config=101, T=T, H=H, I=I, E=E, k=k, fp8=fp8, routing="concentrated")
    ids_ref, w_ref = L.oracle_routing()
    ref = L.oracle_tokens(ids_ref, w_ref, sample_tokens(T, 10 ** 6))
    ws = fm.workspace(L.shape)
    for tr in (16, 32):
        for s1 in (1, 2, 4):
            for s2 in (1, 2, 4):
                for lt in (1, 8):
                    out, ids, _ = fm.fmoe_forward(L.shape, L.x_gpu, L.logits_gpu, L.w, ws=ws, return_routing=True,
                                                  plan=fm.fmoe_plan(tr, s1, s2, lt))
                    assert np.array_equal(ids.cpu().numpy(), ids_ref)
                    st = fm.fmoe_read_stats(ws)
                    # an expert holds at most T = 130 rows: 8 light tiles of 32 rows cover it
                    light_only = lt == 8 and T <= 8 * tr
                    assert st["tile_rows"] == tr and (st["heavy_tiles"] == 0) == light_only
                    assert st["m_tiles"] - st["heavy_tiles"] >= (st["max_rows"] + tr - 1) // tr
                    err = row_rel_err(out.float().cpu().numpy(), ref)
                    assert err <= (FP8_TOL if fp8 else BF16_TOL), f"plan ({tr}, {s1}, {s2}, {lt}): {err:.3e}"


# Up to 16 tokens the forward routes and groups in one launch (wavefront t routes token t and
# the same workgroup then groups the ids from LDS: one wavefront for up to 64 assignments, the
# whole workgroup above).  Its routing must equal the router kernel's bit for bit, its grouping
# the grouping kernel's (same stats, identical output of fmoe_experts on the same ids), and the
# output the oracle's; from T = 17 on the forward takes the two-launch path, held to the same.
@pytest.mark.parametrize("T,H,I,E,k,ep,fp8,scoring,fp32", [
    (1, 256, 128, 128, 8, 1, False, "softmax", False),
    (3, 256, 256, 400, 6, 8, True, "sigmoid", False),    # E > 256: 8 slots per lane; rank 7 of 8
    (16, 512, 256, 64, 8, 1, False, "sigmoid", True),    # fp32 logits
    (16, 256, 128, 1000, 64, 2, False, "softmax", False),  # 16 slots, k = 64: 16 chunks of 64
    (4, 256, 128, 1000, 16, 2, False, "sigmoid", False),   # 64 assignments, one wavefront groups; rank 1 of 2
    (17, 256, 128, 64, 8, 1, False, "softmax", False),   # one past the fused limit
    (32, 256, 128, 64, 8, 1, False, "softmax", False),   # 256 assignments, 32-row light tiles
    (64, 256, 128, 16, 4, 1, False, "sigmoid", True),    # heavy launch possible
    (40, 256, 256, 32, 2, 1, True, "softmax", False),    # FP8: several light tiles per expert allowed
])
def test_small_batch_fused_router_and_grouping(T, H, I, E, k, ep, fp8, scoring, fp32):
    announce(f"fused router+grouping T={T} H={H} I={I} E={E} k={k} ep={ep} fp8={fp8} {scoring} fp32={fp32}")
    L = Layer(config=95, T=T, H=H, I=I, E=E, k=k, fp8=fp8, ep_size=ep, ep_rank=ep - 1, scoring=scoring)
    lg = L.logits.clone()
    lg[T // 2] = float("nan")  # one padding row
    L.logits, L.logits_gpu = lg, (lg.float() if fp32 else lg).cuda()
    ws = fm.workspace(L.shape)
    out, ids, wts = L.forward(ws)
    st_fwd = fm.fmoe_read_stats(ws)
    sc = fm.FMOE_SOFTMAX if scoring == "softmax" else fm.FMOE_SIGMOID
    ids_r, wts_r = fm.fmoe_router_topk(L.logits_gpu, k, sc, True)
    assert torch.equal(ids, ids_r) and torch.equal(wts, wts_r)
    assert ids[T // 2].tolist() == list(range(k))
    out_e = fm.fmoe_experts(L.shape, L.x_gpu, ids, wts, L.w, ws=ws)
    assert fm.fmoe_read_stats(ws) == st_fwd
    assert torch.equal(out_e, out)
    check_layer(L, n_sample=10 ** 6)


# Heavy row tiles of every staged size checked on every token: caller ids give experts of
# 17..513 rows (one to three heavy tiles of 1..4 staged 64-row groups), ragged and empty experts.
@pytest.mark.parametrize("fp8", [False, True])
def test_heavy_tiles_of_every_size_on_every_token(fp8):
    announce(f"heavy tiles of 17..513 rows on every token, fp8={fp8}")
    counts = [0, 1, 15, 16, 17, 31, 32, 33, 64, 65, 128, 129, 256, 257, 300, 513]
    T, H, I, E, k = 470, 512, 384, 16, 4
    flat = np.concatenate([np.full(c, e, np.int32) for e, c in enumerate(counts)])
    pad = np.full(T * k - len(flat), -1, np.int32)
    ids = np.random.default_rng(7).permutation(np.concatenate([flat, pad])).reshape(T, k)
    L = Layer(config=112, T=T, H=H, I=I, E=E, k=k, fp8=fp8)
    wts = np.random.default_rng(8).random((T, k)).astype(np.float32)
    ws = fm.workspace(L.shape)
    out = fm.fmoe_experts(L.shape, L.x_gpu, torch.from_numpy(ids).cuda(), torch.from_numpy(wts).cuda(), L.w, ws=ws)
    st = fm.fmoe_read_stats(ws)
    assert st["local_rows"] == sum(counts) and st["heavy_tiles"] >= 12
    ref = L.oracle_tokens(ids, wts.astype(np.float64), np.arange(T, dtype=np.int32))
    err = row_rel_err(out.float().cpu().numpy(), ref)
    assert err <= (FP8_TOL if fp8 else BF16_TOL), f"{err:.3e}"
