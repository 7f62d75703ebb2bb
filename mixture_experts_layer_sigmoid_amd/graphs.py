"""HIP-graph capture of fmoe_forward at padded token buckets.

Serving calls the layer with a token count that changes from step to step, while a captured
graph needs fixed shapes.  BucketedForward keeps, per bucket size B (the smallest configured
bucket >= T), static buffers of B rows and one HIP graph of an fmoe_forward call on them.  A
call copies the T real rows of x and of the router logits in, sets rows T..B-1 of both to NaN,
replays the graph and returns views of the first T rows of the static outputs.

NaN padding rows are the case of "PR #39593: [Bug]: Fix FlashInfer CUTLASS BF16 + CUDA graphs
IMA", Root cause: under CUDA graphs with data parallelism every rank pads its batch to one size,
and the padding rows carry NaN into the router.  The router replaces NaN by -FLT_MAX and still
picks k distinct experts (the lowest indices), so the padding rows cost some work in experts
0..k-1, and every kernel treats rows independently (the FP8 activation quantizer gives every
row its own scales), so they cannot change a real row.

Everything here is plumbing around the library's entry point: torch copies and fills of the
static buffers, and torch.cuda.CUDAGraph capture and replay.  Every step of the layer runs in
the library's kernels.
"""
from __future__ import annotations

import torch

from . import FMOE_SOFTMAX, ExpertWeights, fmoe_forward, make_shape, workspace

DEFAULT_BUCKETS = (1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048, 4096)


class BucketedForward:
    """fmoe_forward for any T up to the largest bucket, each bucket captured once as a HIP graph.

    The returned tensors are views of static buffers that the next call on the same bucket
    overwrites; copy them to keep them.  One instance serves one device and one weight set;
    calls must not overlap (they share the static buffers and the workspace of a bucket).
    """

    def __init__(self, hidden: int, inter: int, experts: int, top_k: int, weights: ExpertWeights, *,
                 fp8: bool = False, ep_size: int = 1, ep_rank: int = 0, scoring: int = FMOE_SOFTMAX,
                 renormalize: bool = True, logits_dtype=torch.bfloat16, buckets=DEFAULT_BUCKETS,
                 device="cuda"):
        if not buckets or any(b <= 0 for b in buckets):
            raise ValueError("buckets must be positive token counts")
        self.H, self.I, self.E, self.k = hidden, inter, experts, top_k
        self.w = weights
        self.fp8, self.ep_size, self.ep_rank = fp8, ep_size, ep_rank
        self.scoring, self.renormalize = scoring, renormalize
        self.logits_dtype = logits_dtype
        self.buckets = tuple(sorted(set(int(b) for b in buckets)))
        self.device = torch.device(device)
        self._entries: dict[int, dict] = {}

    def bucket(self, tokens: int) -> int:
        for b in self.buckets:
            if b >= tokens:
                return b
        raise ValueError(f"{tokens} tokens exceed the largest bucket ({self.buckets[-1]})")

    def _entry(self, B: int) -> dict:
        e = self._entries.get(B)
        if e is not None:
            return e
        dev = self.device
        e = dict(
            x=torch.full((B, self.H), float("nan"), dtype=torch.bfloat16, device=dev),
            logits=torch.full((B, self.E), float("nan"), dtype=self.logits_dtype, device=dev),
            out=torch.empty((B, self.H), dtype=torch.bfloat16, device=dev),
            ids=torch.empty((B, self.k), dtype=torch.int32, device=dev),
            wts=torch.empty((B, self.k), dtype=torch.float32, device=dev),
            shape=make_shape(B, self.H, self.I, self.E, self.k, self.ep_size, self.ep_rank, self.fp8),
        )
        e["ws"] = workspace(e["shape"], dev)

        def call():
            return fmoe_forward(e["shape"], e["x"], e["logits"], self.w, self.scoring, self.renormalize,
                                ws=e["ws"], out=e["out"], routing_out=(e["ids"], e["wts"]))

        # one eager call first (the library caches device properties on its first launches),
        # on a side stream as graph capture expects, then the capture
        side = torch.cuda.Stream(device=dev)
        side.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(side):
            call()
        torch.cuda.current_stream(dev).wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            call()
        e["graph"] = graph
        self._entries[B] = e
        return e

    def __call__(self, x: torch.Tensor, logits: torch.Tensor, return_routing: bool = False):
        """out [T,H] (and ids [T,k], weights [T,k] when return_routing), as views."""
        T = x.shape[0]
        if x.dim() != 2 or x.shape[1] != self.H or logits.shape != (T, self.E):
            raise ValueError("x must be [T, hidden] and logits [T, experts]")
        if T == 0:
            out = torch.empty((0, self.H), dtype=torch.bfloat16, device=self.device)
            if return_routing:
                return (out, torch.empty((0, self.k), dtype=torch.int32, device=self.device),
                        torch.empty((0, self.k), dtype=torch.float32, device=self.device))
            return out
        e = self._entry(self.bucket(T))
        e["x"][:T].copy_(x)
        e["logits"][:T].copy_(logits)
        if T < e["x"].shape[0]:
            e["x"][T:].fill_(float("nan"))
            e["logits"][T:].fill_(float("nan"))
        e["graph"].replay()
        if return_routing:
            return e["out"][:T], e["ids"][:T], e["wts"][:T]
        return e["out"][:T]
