"""Parity on seeded random shapes: every stage, the grouping by expert and
(on alternate cases) fp8 plus cached dispatch, compared with the oracle on
24 configurations drawn from a fixed seed -- token counts around the
64-token chunk boundaries, 1 to 64 ranks (with 3- and 5-node layouts),
1 to 32 local experts, topk up to 32, 1 to 49 channels, rows of 8 to 1024
elements, expert alignments, masked and duplicate ids, and now and then a
receive capacity a few rows short.  Eight more configurations take dispatch's
pull form: 2048 to 4100 tokens (ragged 128-token groups), rows of 512 to 7168
elements (ragged last tasks), 1 to 64 ranks, a capacity 500 rows short.  Eight
more go through the dispatch straight into the grouped layout at the same token
counts (its pull form for rows of 1 KiB or more and up to 2048 experts), with
topk up to 32, alignment padding, short receive and grouped capacities, and fp8
rows with up to 896 scales per token."""
import numpy as np
import pytest

import gpu_harness as H
import oracle
from test_gpu_parity import _dispatch_grouped_case, _exact, _fp8_case, _group_case, _group_diff, _random_case

pytestmark = pytest.mark.gpu

CASES = 24


def draw(case: int) -> dict:
    rng = np.random.default_rng(4000 + case)
    R = int(rng.choice([1, 2, 4, 8, 16, 24, 32, 40, 64]))
    er = int(rng.choice([1, 2, 3, 4, 8, 16, 32]))
    E = R * er
    K = int(rng.integers(1, min(8, E) + 1))
    if case % 7 == 3:
        K = int(min(E, rng.integers(9, 33)))
    return dict(
        T=int(rng.choice([1, 2, 63, 64, 65, 127, 200, 333, 511, 700])), R=R, E=E, K=K,
        C=int(rng.integers(1, 50)), H=int(rng.choice([16, 64, 256, 1024] if case % 2 == 0 else [8, 24, 200, 520])),
        align=int(rng.choice([1, 2, 4, 16])), mask=float(rng.choice([0.0, 0.0, 0.1, 0.5])),
        dup=bool(case % 3 == 1), short=bool(case % 5 == 2))


@pytest.mark.parametrize("case", range(CASES))
def test_random_shape(case):
    s = draw(case)
    print(f"[parity] random case {case}: {s}", flush=True)
    x, idx, w = _random_case(s["T"], s["R"], s["E"], s["K"], s["C"], s["H"], seed=5000 + case, mask_frac=s["mask"],
                             dup=s["dup"])
    n = int(oracle.Oracle().layout(idx, s["E"], s["R"])["num_tokens_per_rank"].sum())
    cap = max(0, n - 3) if s["short"] else None
    gpu, ref = H.run_both(x, idx, w, s["E"], s["R"], s["C"], align=s["align"], capacity=cap)
    assert H.compare(gpu, ref) == []
    assert H.combine_bit_differences(gpu, ref) == {"combined_x": 0}
    assert gpu["dev_status"] == ref["status"]
    g, want = _group_case(x, idx, w, s["E"], s["R"], s["C"], s["align"])
    assert _group_diff(g, want) == []
    if case % 2 == 0:  # rows of whole 16-byte units as fp8 (H % 16 == 0), 8-element scale blocks
        g8, r8 = _fp8_case(x, idx, w, s["E"], s["R"], s["C"], num_scales_block=8, capacity=cap)
        assert _exact(g8, r8) == []
        assert g8["status"] == r8["status"]


PULL_CASES = 8


def draw_pull(case: int) -> dict:
    """Shapes that take dispatch's pull form: 2048 tokens or more (ragged 128-token
    groups), rows of 1 KiB or more, ragged last tasks of a row."""
    rng = np.random.default_rng(6000 + case)
    R = int(rng.choice([1, 8, 16, 24, 32, 64]))
    er = int(rng.choice([1, 2, 4, 8]))
    E = R * er
    K = int(rng.integers(1, min(8, E) + 1))
    return dict(
        T=int(rng.choice([2048, 2049, 2111, 2176, 3000, 4100])), R=R, E=E, K=K, C=int(rng.integers(1, 40)),
        H=int(rng.choice([512, 520, 1000, 2056, 3592, 7168])), align=int(rng.choice([1, 4, 8])),
        mask=float(rng.choice([0.0, 0.2])), dup=bool(case % 3 == 1), short=bool(case % 4 == 2))


@pytest.mark.parametrize("case", range(PULL_CASES))
def test_random_shape_pull(case):
    s = draw_pull(case)
    print(f"[parity] random pull case {case}: {s}", flush=True)
    x, idx, w = _random_case(s["T"], s["R"], s["E"], s["K"], s["C"], s["H"], seed=7000 + case, mask_frac=s["mask"],
                             dup=s["dup"])
    n = int(oracle.Oracle().layout(idx, s["E"], s["R"])["num_tokens_per_rank"].sum())
    cap = max(0, n - 500) if s["short"] else None
    gpu, ref = H.run_both(x, idx, w, s["E"], s["R"], s["C"], align=s["align"], capacity=cap)
    assert H.compare(gpu, ref) == []
    assert H.combine_bit_differences(gpu, ref) == {"combined_x": 0}
    assert gpu["dev_status"] == ref["status"]
    g, want = _group_case(x, idx, w, s["E"], s["R"], s["C"], s["align"])
    assert _group_diff(g, want) == []
    if case % 2 == 0 and s["H"] % 16 == 0:  # fp8 rows of whole 16-byte units, 8-element scale blocks
        g8, r8 = _fp8_case(x, idx, w, s["E"], s["R"], s["C"], num_scales_block=8, capacity=cap)
        assert _exact(g8, r8) == []
        assert g8["status"] == r8["status"]


GROUPED_CASES = 8


def draw_grouped(case: int) -> dict:
    """Shapes for the dispatch straight into the grouped layout at 2048 tokens or more."""
    rng = np.random.default_rng(8000 + case)
    R = int(rng.choice([1, 8, 16, 24, 32, 64]))
    er = int(rng.choice([1, 2, 4, 8, 16, 32]))
    E = R * er
    K = int(rng.integers(1, min(8, E) + 1))
    if case % 4 == 3:
        K = int(min(E, rng.integers(9, 33)))
    return dict(
        T=int(rng.choice([2048, 2049, 2111, 2176, 3000, 4100])), R=R, E=E, K=K, C=int(rng.integers(1, 40)),
        H=int(rng.choice([512, 520, 1000, 2056, 3592, 7168])), align=int(rng.choice([1, 2, 4, 16])),
        mask=float(rng.choice([0.0, 0.2])), dup=bool(case % 3 == 1),
        recv_delta=-300 if case % 4 == 2 else 0, gcap_delta=-200 if case % 4 == 1 else 0)


@pytest.mark.parametrize("case", range(GROUPED_CASES))
def test_random_shape_grouped_pull(case):
    s = draw_grouped(case)
    print(f"[parity] random grouped case {case}: {s}", flush=True)
    x, idx, w = _random_case(s["T"], s["R"], s["E"], s["K"], s["C"], s["H"], seed=9000 + case, mask_frac=s["mask"],
                             dup=s["dup"])
    gpu, want = _dispatch_grouped_case(x, idx, w, s["E"], s["R"], s["C"], s["align"], recv_delta=s["recv_delta"],
                                       gcap_delta=s["gcap_delta"])
    assert _group_diff(gpu, want) == []
    if case % 2 == 0 and s["H"] % 16 == 0:  # fp8 rows of whole 16-byte units, 8-element scale blocks
        g8, w8 = _dispatch_grouped_case(x, idx, w, s["E"], s["R"], s["C"], s["align"], fp8=True, scale_block=8)
        assert _group_diff(g8, w8) == []
