"""The down GEMM and the combine in one launch (bf16, at most 64 assignments): every token of
every case against the oracle, against the two-launch path (the same call with the reduction
splits set by a plan), and bit for bit against itself on repeated calls.

Cases: the 2048 x 768, 128-expert top-8 layer at 1..8 tokens (uniform and concentrated), every
count of 16-byte pieces per lane (I = 128 .. 1024, ragged ones included: I = 384 leaves half of
the second piece's lanes past the row end), expert-parallel shards whose tokens may have no
local expert (zero rows), caller ids with repeats (an expert of 64 rows is cut into heavy
tiles, which the fused launch walks after the light ones) and ids outside [0, E), and the
64-assignment limit on both sides."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_sigmoid_amd as fm
import oracle
from mixture_experts_layer_sigmoid_amd import synth
from gpu_common import BF16_TOL, Layer, announce, check_layer, row_rel_err

pytestmark = pytest.mark.gpu


def split_plan():
    p = fm.fmoe_plan()
    p.split_gate_up = 2  # a down split in the plan keeps the down GEMM and the combine apart
    p.split_down = 2
    return p


def two_paths(L: Layer):
    fused, ids, _ = L.forward()
    L.plan = split_plan()
    plain, ids2, _ = L.forward()
    L.plan = None
    torch.cuda.synchronize()
    assert torch.equal(ids, ids2)
    return fused.float().cpu().numpy(), plain.float().cpu().numpy()


@pytest.mark.parametrize("T", [1, 2, 3, 5, 8])
@pytest.mark.parametrize("routing", ["uniform", "concentrated"])
def test_fused_down_combine_2048x768_e128_top8(T, routing):
    announce(f"down+combine: 2048x768 E128 top8 T={T} {routing}")
    L = Layer(config=3, T=T, H=2048, I=768, E=128, k=8, routing=routing, seed=T)
    check_layer(L, n_sample=T)
    fused, plain = two_paths(L)
    assert row_rel_err(fused, plain) <= BF16_TOL


@pytest.mark.parametrize("I", [128, 256, 384, 512, 640, 768, 896, 1024])
def test_fused_down_combine_every_piece_count(I):
    announce(f"down+combine: I={I}")
    L = Layer(config=96, T=7, H=384, I=I, E=16, k=4, seed=I)
    check_layer(L, n_sample=7)


@pytest.mark.parametrize("H", [128, 256, 640, 1280, 1664, 2048, 2560])
def test_fused_down_combine_every_hidden_size(H):
    announce(f"down+combine: H={H} (H/8 workgroups)")
    L = Layer(config=94, T=5, H=H, I=256, E=16, k=4, seed=H)
    check_layer(L, n_sample=5)
    fused, plain = two_paths(L)
    assert row_rel_err(fused, plain) <= BF16_TOL


@pytest.mark.parametrize("ep_rank", [0, 3, 7])
def test_fused_down_combine_expert_shard(ep_rank):
    announce(f"down+combine: EP shard rank {ep_rank} of 8, T=6")
    L = Layer(config=97, T=6, H=512, I=256, E=32, k=4, ep_size=8, ep_rank=ep_rank, seed=ep_rank)
    check_layer(L, n_sample=6)


def test_fused_down_combine_no_local_rows_gives_zeros():
    announce("down+combine: shard without a local assignment")
    T, H, I, E, k = 4, 256, 128, 16, 2
    L = Layer(config=98, T=T, H=H, I=I, E=E, k=k, ep_size=4, ep_rank=3, seed=1)
    ids = torch.zeros((T, k), dtype=torch.int32, device="cuda")
    ids[:, 1] = 1  # every pick on experts 0 and 1, which rank 3 does not hold
    wts = torch.full((T, k), 0.5, dtype=torch.float32, device="cuda")
    out = torch.full((T, H), 7.0, dtype=torch.bfloat16, device="cuda")
    fm.fmoe_experts(L.shape, L.x_gpu, ids, wts, L.w, out=out)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0


@pytest.mark.parametrize("case", ["one_expert", "out_of_range"])
def test_fused_down_combine_caller_ids_heavy_tiles_and_dropped(case):
    T, H, I, E, k = 16, 256, 128, 8, 4  # 64 assignments: the largest fused batch
    announce(f"down+combine: caller ids, {case}, n={T * k}")
    L = synth.tiny_layer(T, H, E, I, seed=11)
    w = fm.ExpertWeights(L["wg"].cuda(), L["wu"].cuda(), L["wd"].cuda())
    shape = fm.make_shape(T, H, I, E, k)
    g = np.random.default_rng(3)
    if case == "one_expert":
        ids = np.full((T, k), 5, np.int32)  # 64 rows on expert 5: heavy tiles
    else:
        ids = g.integers(-2, E + 2, (T, k)).astype(np.int32)
    wts = g.random((T, k)).astype(np.float32)
    ws = fm.workspace(shape)
    out = fm.fmoe_experts(shape, L["x"].cuda(), torch.from_numpy(ids).cuda(), torch.from_numpy(wts).cuda(), w, ws=ws)
    torch.cuda.synchronize()
    bits = [synth.bf16_bits(L[n]) for n in ("wg", "wu", "wd")]
    ref = oracle.moe_tokens(synth.bf16_bits(L["x"]), ids, wts.astype(np.float64), *bits, E=E)
    assert row_rel_err(out.float().cpu().numpy(), ref) <= BF16_TOL
    st = fm.fmoe_read_stats(ws)
    if case == "one_expert":
        assert st["heavy_tiles"] >= 1 and st["max_rows"] == T * k
    else:
        assert st["dropped_ids"] == int(((ids < 0) | (ids >= E)).sum())


@pytest.mark.parametrize("T,k", [(8, 8), (13, 5), (16, 4), (17, 4)])
def test_fused_down_combine_limit(T, k):
    announce(f"down+combine limit: T={T} k={k} (n={T * k})")
    L = Layer(config=99, T=T, H=256, I=384, E=16, k=k, seed=T)
    check_layer(L, n_sample=T)


def test_fused_down_combine_is_deterministic():
    announce("down+combine: 20 repeated calls bit-equal")
    L = Layer(config=3, T=4, H=2048, I=768, E=128, k=8, seed=4)
    first, _, _ = L.forward()
    for _ in range(20):
        again, _, _ = L.forward()
        assert torch.equal(first, again)


def test_fused_down_combine_top2_of_32_tokens():
    # 32 tokens of top-2: 64 assignments, one or two rows for most experts
    announce("down+combine: T=32 H=1280 k=2")
    L = Layer(config=93, T=32, H=1280, I=256, E=16, k=2, seed=32)
    check_layer(L, n_sample=32)
