"""The algorithmic byte counts bench.py divides by (CPU only).

They follow the definition of what each stage must move: x read once per token,
the ids and weights read, every receive row written with its metadata, the
send_slot map; combine the reverse.  Pinned to reference figures worked out
from that definition by hand at each workload's expected receive-row count
(E[N] = R * (1 - C(E - E/R, k) / C(E, k)) per token for uniform routing, a
seeded sample for the skewed one), to a buffer-by-buffer count, and to the
committed rocprofv3 counter summary (measured HBM bytes within 2%).
"""
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

# (t, h, k, R, expected N) -> (dispatch MB, combine MB), MB = 1e6 bytes, one decimal
TABLE = {
    "sweep": ((128, 7168, 8, 16, 835), (13.9, 13.8)),
    "prefill": ((4096, 7168, 8, 64, 31440), (514.2, 511.6)),
    "skew": ((4096, 7168, 8, 32, 25252), (424.3, 422.2)),
    "large": ((16384, 4096, 6, 16, 87100), (856.9, 851.3)),
}


@pytest.mark.parametrize("name", sorted(TABLE))
def test_bytes_match_the_tabulated_figures(name):
    (T, H, K, R, N), (d_mb, c_mb) = TABLE[name]
    assert round(bench.dispatch_bytes(T, H, K, R, N) / 1e6, 1) == pytest.approx(d_mb, abs=0.051)
    assert round(bench.combine_bytes(T, H, K, R, N) / 1e6, 1) == pytest.approx(c_mb, abs=0.051)


def test_bytes_are_the_buffers_moved():
    # count each buffer from its shape and dtype (bf16 rows, i64 ids, f32 weights, i32 maps)
    T, H, K, R, N, S, M = 300, 512, 6, 16, 1234, 4, 1500
    nb = lambda shape, dt: int(np.prod(shape)) * np.dtype(dt).itemsize  # noqa: E731
    x, idx, w = nb((T, H), np.int16), nb((T, K), np.int64), nb((T, K), np.float32)
    recv_x, recv_w, recv_idx, src = nb((N, H), np.int16), nb((N, K), np.float32), nb((N, K), np.int64), nb((N, 2), np.int32)
    slot = nb((T, R), np.int32)
    out, out_w = nb((T, H), np.int16), nb((T, K), np.float32)
    assert bench.dispatch_bytes(T, H, K, R, N) == x + idx + w + recv_x + recv_w + recv_idx + src + slot
    assert bench.combine_bytes(T, H, K, R, N) == recv_x + recv_w + slot + out + out_w
    x8, sc = nb((T, H), np.uint8), nb((T, S), np.float32)
    r8, rsc = nb((N, H), np.uint8), nb((N, S), np.float32)
    assert bench.dispatch_fp8_bytes(T, H, K, R, N, S) == x8 + sc + idx + w + r8 + rsc + recv_w + recv_idx + src + slot
    assert bench.dispatch_cached_bytes(T, R, N, 2 * H, 0) == x + slot + recv_x
    assert bench.quantize_bytes(T, H, S) == x + x8 + sc
    assert bench.dequantize_bytes(N, H, S) == r8 + rsc + recv_x
    assert bench.dispatch_cached_to_fp8_bytes(T, H, R, N, S) == x + slot + r8 + rsc
    assert bench.dispatch_to_fp8_bytes(T, H, K, R, N, S) == x + idx + w + r8 + rsc + recv_w + recv_idx + src + slot
    g_x, g_row, g_w, pos = nb((M, H), np.int16), nb((M,), np.int32), nb((M,), np.float32), nb((N, K), np.int32)
    assert bench.group_bytes(H, K, N, M) == recv_x + recv_idx + recv_w + g_x + g_row + g_w + pos
    assert bench.dispatch_grouped_bytes(T, H, K, R, N, M) == (x + idx + w + slot + recv_w + recv_idx + src + pos
                                                              + g_x + g_row + g_w)


def test_committed_counters_agree_with_the_algorithmic_bytes():
    fields = {}
    with open(bench.PROFILE) as fh:
        for line in fh:
            parts = line.split()
            if len(parts) == 7 and parts[-1].isdigit():
                fields[parts[0]] = (int(parts[5]), int(parts[6]))
    # the prefill workload's dispatch and combine kernels (rows of 14 KiB from 4096 tokens)
    for kernel in ("dispatch_pull_kernel", bench.combine_kernel_name(4096, 7168)):
        traffic, algorithmic = fields[kernel]
        assert abs(traffic - algorithmic) / algorithmic < 0.02, (kernel, traffic, algorithmic)
