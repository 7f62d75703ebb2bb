"""GPU parity of the per-expert grouping: counts, offsets, the stable permutation and its
inverse bit-exact against the oracle; counters; determinism."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_sigmoid_amd as fm
import oracle
from mixture_experts_layer_sigmoid_amd import synth
from gpu_common import announce

pytestmark = pytest.mark.gpu


def check_group(ids: np.ndarray, E: int, ep_size=1, ep_rank=0, H=256, I=128, fp8=False):
    T, k = ids.shape
    shape = fm.make_shape(T, H, I, E, k, ep_size, ep_rank, fp8=fp8)
    r = fm.fmoe_route_permute(shape, torch.from_numpy(np.ascontiguousarray(ids, np.int32)).cuda())
    ref = oracle.route_permute(ids, E, ep_size, ep_rank)
    R = int(ref["offsets"][-1])
    assert np.array_equal(r["counts"].cpu().numpy(), ref["counts"])
    assert np.array_equal(r["offsets"].cpu().numpy(), ref["offsets"])
    assert np.array_equal(r["perm_src"].cpu().numpy()[:R], ref["perm_src"])
    assert np.array_equal(r["inv_perm"].cpu().numpy(), ref["inv_perm"])
    st = fm.fmoe_read_stats(r["ws"])
    assert st["local_rows"] == R
    assert st["dropped_ids"] == ref["dropped"]
    assert st["max_rows"] == int(ref["counts"].max(initial=0))
    assert st["empty_experts"] == int((ref["counts"] == 0).sum())
    est = max(1, -(-T * k // E))
    assert st["rows_estimate"] == est
    tr = st["tile_rows"]
    # light tile: 16 rows at one expected row, 32 from two on; from 32 expected rows on, the
    # smallest again (every expert above 16 rows goes to the heavy-tile kernel)
    assert tr == (16 if est == 1 or est >= 32 else 32)
    # FP8: caller ids may repeat, so an expert can hold up to T*k rows; when that fits 8 light
    # tiles, every expert is cut into light tiles of tr rows and there are no heavy tiles
    cap = 8 * tr if fp8 and T * k <= 8 * tr else tr
    heavy_counts = [int(c) for c in ref["counts"] if c > cap]
    # heavy experts: ceil(c / 256) tiles of about equal size; bf16 experts of 257..320 rows are
    # one tile when the 256-row tiles give each compute unit four tasks in the GEMM with the
    # fewer 128-column blocks
    n256 = sum(-(-c // 256) for c in heavy_counts)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    nb = min(2 * I // 128, H // 128)
    five = not fp8 and n256 >= -(-4 * cus // nb)
    assert st["heavy_rows"] == (320 if five else 256)
    heavy = sum(1 if five and 256 < c <= 320 else -(-c // 256) for c in heavy_counts)
    light = int(sum(-(-c // tr) for c in ref["counts"] if 0 < c <= cap))
    assert st["heavy_tiles"] == heavy
    assert st["m_tiles"] == light + heavy
    return r, ref


@pytest.mark.parametrize("T,k,E,ep_size,ep_rank", [
    (1, 1, 1, 1, 0), (1, 8, 128, 1, 0), (37, 3, 16, 1, 0), (64, 8, 128, 1, 0), (300, 4, 8, 1, 0),
    (288, 6, 400, 8, 0), (288, 6, 400, 8, 5), (513, 8, 64, 4, 3), (4096, 8, 128, 1, 0), (2000, 2, 1024, 1, 0),
    (512, 8, 128, 1, 0), (1024, 4, 16, 1, 0), (1040, 4, 16, 2, 1),  # 64 chunks (one launch), 65 chunks
    # from 256 chunks on, blocks of 8 chunks: a ragged last block and chunk, 1024 local experts,
    # an expert-parallel rank
    (2083, 8, 128, 1, 0), (4100, 4, 1024, 1, 0), (4133, 7, 400, 8, 5),
])
@pytest.mark.parametrize("fp8", [False, True])  # FP8: several light tiles per expert where they bound it
def test_group_random_ids_with_duplicates(T, k, E, ep_size, ep_rank, fp8):
    announce(f"group T={T} k={k} E={E} ep={ep_size}/{ep_rank} fp8={fp8}")
    g = np.random.default_rng(T * 7 + E)
    ids = g.integers(0, E, (T, k)).astype(np.int32)  # repeated ids in a token are legal
    check_group(ids, E, ep_size, ep_rank, fp8=fp8)


def test_group_router_ids_full_sizes():
    # the 128-expert layer (H=2048, I=768) at T=4096: under uniform routing about half the experts
    # hold 257..320 rows, one tile each
    for cfg, T, E, k, routing, ep, H, I in [(3, 4096, 128, 8, "uniform", 1, 2048, 768),
                                            (3, 4096, 128, 8, "concentrated", 1, 2048, 768),
                                            (3, 4096, 128, 8, "uniform", 1, 256, 128),
                                            (5, 288, 400, 6, "uniform", 8, 7168, 2048),
                                            (5, 288, 400, 6, "concentrated", 8, 7168, 2048)]:
        announce(f"group router ids T={T} E={E} k={k} {routing} ep={ep} H={H} I={I}")
        lg = synth.routed_logits(cfg, T, E, k, routing)
        ids, _ = oracle.router_topk(synth.bf16_bits(lg), k)
        r, ref = check_group(ids, E, ep, 0, H=H, I=I)
        if (H, routing) == (2048, "uniform"):
            st = fm.fmoe_read_stats(r["ws"])
            assert st["heavy_rows"] == 320 and st["heavy_tiles"] < int((ref["counts"] > 256).sum()) + 128
        if routing == "concentrated":
            hot = ref["counts"][:8].sum()
            assert hot >= 0.85 * T * k


def test_group_all_tokens_one_expert_and_out_of_range():
    announce("group all tokens to one expert, out-of-range ids")
    T, k, E = 200, 6, 32
    check_group(np.zeros((T, k), np.int32), E)
    g = np.random.default_rng(3)
    ids = g.integers(-5, E + 5, (T, k)).astype(np.int32)
    check_group(ids, E)
    check_group(ids, E, 4, 2)


def test_group_is_deterministic():
    announce("group determinism")
    T, k, E = 4096, 8, 128
    ids = torch.from_numpy(np.random.default_rng(5).integers(0, E, (T, k)).astype(np.int32)).cuda()
    shape = fm.make_shape(T, 2048, 768, E, k)
    first = fm.fmoe_route_permute(shape, ids)
    for _ in range(10):
        again = fm.fmoe_route_permute(shape, ids)
        for key in ("counts", "offsets", "perm_src", "inv_perm"):
            assert torch.equal(again[key], first[key])
