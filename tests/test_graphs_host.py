"""Bucket choice of the graph helper (host logic, no GPU)."""
import pytest

from mixture_experts_layer_sigmoid_amd.graphs import DEFAULT_BUCKETS, BucketedForward


def test_bucket_is_the_smallest_that_fits():
    bf = BucketedForward(256, 128, 8, 2, weights=None, buckets=(64, 8, 1, 8))
    assert bf.buckets == (1, 8, 64)
    assert [bf.bucket(t) for t in (1, 2, 8, 9, 64)] == [1, 8, 8, 64, 64]
    with pytest.raises(ValueError):
        bf.bucket(65)
    assert BucketedForward(256, 128, 8, 2, weights=None).bucket(4096) == DEFAULT_BUCKETS[-1]
    with pytest.raises(ValueError):
        BucketedForward(256, 128, 8, 2, weights=None, buckets=(0, 4))
