"""The pool-placement helpers: shapes, contiguity, non-overlap, and the 256-byte phase of
the second pool against the first (checked on CPU tensors; the same arithmetic holds on the
GPU, where the GPU tests run the paged workloads laid out this way)."""

import pytest
import torch

from top_kv_block_amd import qsparse as qs
from top_kv_block_amd import workloads as W


@pytest.mark.parametrize("shape,dtype", [((7, 16, 2, 128), torch.bfloat16), ((3, 32, 8, 128), torch.float32),
                                         ((1, 128, 1, 128), torch.float16), ((5, 16, 3, 128), torch.int8)])
@pytest.mark.parametrize("make", ["binding", "workloads"])
def test_paired_pools_phase(shape, dtype, make):
    a, b = qs.alloc_paired_pools(shape, dtype, "cpu") if make == "binding" else W.paired_pools(shape, dtype, "cpu")
    for t in (a, b):
        assert t.shape == shape and t.dtype == dtype and t.is_contiguous()
    nbytes = a.numel() * a.element_size()
    delta = b.data_ptr() - a.data_ptr()
    assert delta >= nbytes                      # no overlap
    assert delta % 1024 == 256                  # the second starts 256 B past a 1 KiB multiple
    assert a.data_ptr() % 16 == 0 and b.data_ptr() % 16 == 0
    a.fill_(1)
    b.zero_()
    assert int(a.float().sum()) == a.numel()    # writing one never touches the other


def test_metadata_pools_are_zeroed():
    mx, mn = qs.alloc_metadata_pools(4, 16, 2, 128, torch.bfloat16, "cpu")
    assert mx.shape == (4, 16, 2, 128) and not mx.any() and not mn.any()
    assert (mn.data_ptr() - mx.data_ptr()) % 1024 == 256
    k, v = qs.alloc_kv_pools(6, 32, 4, 128, torch.float32, "cpu")
    assert k.shape == v.shape == (6, 32, 4, 128) and (v.data_ptr() - k.data_ptr()) % 1024 == 256
