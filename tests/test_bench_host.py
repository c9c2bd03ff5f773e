"""Host-side checks of bench.py's bookkeeping (no GPU)."""
import os

import pytest

import bench

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(
    __file__))), "kernelized_attention_scan_amd", "csrc")


def test_kernel_source_lists_name_existing_files():
    for kind, names in bench.KERNEL_SOURCES.items():
        for n in names:
            assert os.path.exists(os.path.join(CSRC, n)), (kind, n)


def test_every_device_source_is_tracked():
    # the one source no timed kernel is built from: the standalone feature map
    tracked = set(sum(bench.KERNEL_SOURCES.values(), [])) | {"la_featmap.hip"}
    assert set(os.listdir(CSRC)) <= tracked


@pytest.mark.parametrize("w,kind", [("decayed", "forward"),
                                    ("performer", "forward"),
                                    ("gated", "forward"),
                                    ("decode", "decode"),
                                    ("backward", "backward")])
def test_kernel_kind(w, kind):
    assert bench.kernel_kind(w) == kind
    assert len(bench.kernel_source_hash(kind)) == 16
