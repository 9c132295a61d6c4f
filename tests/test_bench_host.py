"""Host-side checks of bench.py's bookkeeping (no GPU): every kernel the
roofline may name has a label and a source list, and the source hashes that
tie committed counter runs to kernel versions are computable."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("order", [1, 2])
@pytest.mark.parametrize("dtype", ["f64", "f32"])
@pytest.mark.parametrize("tensorial", [False, True])
def test_contract_kernel_named(order, dtype, tensorial):
    k = bench.contract_kernel(order, dtype, tensorial)
    assert k in bench.KERNEL_FILES and k in bench.KERNEL_LABELS


def test_every_kernel_hashable():
    for k in bench.KERNEL_FILES:
        assert k in bench.KERNEL_LABELS
        h = bench.kernel_source_hash(k)
        assert len(h) == 16 and int(h, 16) >= 0
