"""Builds tests/c/_build/libgsfp8_capped_grid.so: the library with tiny grid
caps (at most 3 workgroups per quantize / dequantize launch, 5 per unscale
launch), so that the grid-stride loops every kernel takes past its cap in
the real build (2^20 workgroups: tensors of several 10^9 elements) run on
small inputs, where the GPU tests compare them with the oracle.

    python tests/c/build_capped_grid.py [OUT]
"""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from loss_scaling_fp8_amd import build as libbuild  # noqa: E402

DEFINES = ["-DGS_MAX_GRID=3", "-DGS_UNSCALE_GRID_CAP=5"]


def build(out=None):
    out = out or os.path.join(HERE, "_build", "libgsfp8_capped_grid.so")
    os.makedirs(os.path.dirname(out), exist_ok=True)
    return libbuild.build_variant(out, DEFINES)


if __name__ == "__main__":
    print(build(sys.argv[1] if len(sys.argv) > 1 else None))
