"""bench.py keys its counter lookups on the launch grids the library uses;
these tests pin its copies of the library's launch rules to grids the
kernel traces of the 5B step show (CPU only)."""
import os
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
bench = pytest.importorskip("bench")

M5B = 17776


def test_int8_workgroup_size():
    # whole rows per workgroup: 192 threads when they leave fewer lanes idle
    assert bench.int8_threads(48) == 192      # K = 3072: 4 rows of 48 chunks
    assert bench.int8_threads(192) == 192     # K = 12288: one row
    assert bench.int8_threads(30) == 256      # K = 1920: 8 rows of 30 (240 of 256 lanes)
    assert bench.int8_threads(120) == 256     # K = 7680: 2 rows
    assert bench.int8_threads(256) == 256
    for cpr in range(1, 257):
        t = bench.int8_threads(cpr)
        assert t in (192, 256) and t // cpr >= 1


def test_quantize_grids_of_the_5b_step():
    for fmt in ("nvfp4", "mxfp4", "mxfp8"):
        assert bench.hq_grid_work_items(M5B, 3072, fmt) == 853248
        assert bench.hq_grid_work_items(M5B, 12288, fmt) == 3412992
    assert bench.hq_grid_work_items(M5B, 3072, "int8") == 853248     # 4444 groups of 192
    assert bench.hq_grid_work_items(M5B, 12288, "int8") == 3412992   # 17776 groups of 192
    assert bench.hq_grid_work_items(106306, 3072, "nvfp4") == 5102720  # 1080p, rounded to 128


def test_gemm_work_split_of_the_5b_step():
    # QKV: 70 x 36 = 2520 tiles, 9.8 waves on 256 CUs, not split
    assert bench.gemm_call_grids(M5B, 9216, 3072) == {"dp": 645120, "sk": 0, "reduce": 0}
    # FFN-down: 840 tiles; the last 72 split into 3 K slices of 32 stages
    assert bench.gemm_call_grids(M5B, 3072, 12288) == {"dp": 196608, "sk": 55296, "reduce": 1179648}
    # out-proj: 840 tiles; 72 tiles in 3 slices of 8 stages
    assert bench.gemm_call_grids(M5B, 3072, 3072) == {"dp": 196608, "sk": 55296, "reduce": 1179648}
    # FFN-up: 3360 tiles; the last 32 in 8 slices of 3 stages
    assert bench.gemm_call_grids(M5B, 12288, 3072) == {"dp": 851968, "sk": 65536, "reduce": 524288}
