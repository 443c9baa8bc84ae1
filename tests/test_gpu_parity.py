"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Layout, notify and dispatch outputs must be bit-exact; combined rows must be
within max |diff| 1e-2 (bf16 outputs, fp32 accumulation), and -- because
both sides reduce in the same order with fp32 fma -- are also checked to be
bit-exact.  The five workloads run at full size, in the launch configuration
the benchmark uses, and the oracle computes every output element."""
import numpy as np
import pytest

import gpu_harness as H
from combine_ep_get_02_amd.inputs import WORKLOADS, generate

pytestmark = pytest.mark.gpu


def _run(name, **kw):
    d = generate(name)
    wl = d["workload"]
    rng = np.random.default_rng(11)
    return H.run_both(d["x"], d["topk_idx"], d["topk_weights"], wl.experts, wl.ranks, wl.channels, **kw), rng


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_workload_parity(name):
    print(f"[parity] workload={name}", flush=True)
    d = generate(name)
    wl = d["workload"]
    rng = np.random.default_rng(11)
    # independent expert outputs y for the second combine; rows count from the oracle's N
    import oracle
    lay = oracle.Oracle().layout(d["topk_idx"], wl.experts, wl.ranks)
    n = int(lay["num_tokens_per_rank"].sum())
    y = H.random_rows(rng, n, wl.hidden)
    gpu, ref = H.run_both(d["x"], d["topk_idx"], d["topk_weights"], wl.experts, wl.ranks, wl.channels, y=y)
    assert H.compare(gpu, ref) == []
    assert H.combine_bit_differences(gpu, ref) == {"combined_x": 0, "combined_x_y": 0}
    assert gpu["dev_status"] == 0 and ref["status"] == 0
    # identity experts return x for every token that went anywhere (as values:
    # the accumulator starts at +0, so an x element of -0 comes back as +0)
    live = ref["is_token_in_rank"].any(1)
    import pins
    assert np.array_equal(pins.bf16_to_f64(gpu["combined_x"][live]), pins.bf16_to_f64(d["x"][live]))


def _random_case(T, R, E, K, C, H_, seed, mask_frac=0.0, dup=False):
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.choice(E, K, replace=dup) for _ in range(T)]).astype(np.int64) if T else \
        np.zeros((0, K), np.int64)
    if mask_frac and T:
        flat = rng.choice(T * K, int(mask_frac * T * K), replace=False)
        idx.reshape(-1)[flat] = -1
    w = rng.random((T, K)).astype(np.float32)
    x = H.random_rows(rng, T, H_)
    return x, idx, w


EDGE = {
    # name: (T, R, E, K, C, H, extra)
    "t_less_than_channels": (3, 8, 16, 2, 7, 64, {}),
    "single_rank": (100, 1, 4, 2, 3, 256, {}),
    "four_ranks_one_node": (200, 4, 8, 3, 5, 512, {}),
    "r24_three_nodes": (300, 24, 48, 4, 6, 128, {}),
    "k1": (257, 16, 32, 1, 4, 7168, {}),
    "k32_r64": (130, 64, 128, 32, 9, 4096, {}),
    "hidden8_ragged_chunks": (1000, 64, 256, 8, 24, 8, {}),
    "hidden800_nonexact": (333, 16, 64, 6, 5, 800, {}),
    "many_channels": (500, 16, 64, 4, 4096, 64, {}),
    "huge_expert_count_global_atomics": (700, 64, 16384, 8, 24, 128, {}),
    "masked_and_duplicates": (400, 32, 256, 8, 24, 256, dict(mask_frac=0.3, dup=True)),
    "fully_masked_tokens": (129, 16, 64, 4, 3, 128, dict(mask_frac=1.0)),
    # 1563 chunks at 64 ranks: the counts do not fit LDS, notify scans in global memory
    "t100k_global_scan": (100000, 64, 256, 8, 24, 64, {}),
    "hidden_32768": (33, 8, 16, 2, 3, 32768, {}),
}


@pytest.mark.parametrize("name", sorted(EDGE))
def test_edge_parity(name):
    T, R, E, K, C, H_, extra = EDGE[name]
    print(f"[parity] edge={name}", flush=True)
    x, idx, w = _random_case(T, R, E, K, C, H_, seed=len(name), **extra)
    rng = np.random.default_rng(5)
    import oracle
    n = int(oracle.Oracle().layout(idx, E, R)["num_tokens_per_rank"].sum())
    y = H.random_rows(rng, n, H_)
    gpu, ref = H.run_both(x, idx, w, E, R, C, y=y)
    assert H.compare(gpu, ref) == []
    assert all(v == 0 for v in H.combine_bit_differences(gpu, ref).values())
    assert gpu["dev_status"] == ref["status"] == 0


def test_empty_tokens():
    x, idx, w = _random_case(0, 16, 64, 4, 8, 64, seed=1)
    gpu, ref = H.run_both(x, idx, w, 64, 16, 8, capacity=0)
    assert H.compare(gpu, ref) == []
    assert gpu["num_recv_tokens"] == 0 and not gpu["gbl_channel_prefix_matrix"].any()


@pytest.mark.parametrize("align", [4, 128])
def test_expert_alignment(align):
    x, idx, w = _random_case(512, 16, 64, 6, 8, 64, seed=align)
    gpu, ref = H.run_both(x, idx, w, 64, 16, 8, align=align)
    assert H.compare(gpu, ref) == []


def test_my_rank_is_src_rank():
    x, idx, w = _random_case(300, 8, 32, 4, 4, 64, seed=9)
    gpu, ref = H.run_both(x, idx, w, 32, 8, 4, my_rank=5)
    assert H.compare(gpu, ref) == []
    assert np.all(gpu["recv_src_info"][:, 0] == 5)


def test_bad_topk_ids_flagged_and_masked():
    x, idx, w = _random_case(300, 16, 64, 4, 4, 64, seed=3)
    idx[5, 1] = 64
    idx[77, 0] = -9
    gpu, ref = H.run_both(x, idx, w, 64, 16, 4)
    assert H.compare(gpu, ref) == []
    assert gpu["dev_status"] & 1 and ref["status"] & 1


def test_receive_capacity_overflow():
    x, idx, w = _random_case(300, 16, 64, 4, 4, 64, seed=4)
    import oracle
    n = int(oracle.Oracle().layout(idx, 64, 16)["num_tokens_per_rank"].sum())
    gpu, ref = H.run_both(x, idx, w, 64, 16, 4, capacity=n - 37)
    assert H.compare(gpu, ref) == []
    assert gpu["dev_status"] & 2 and ref["status"] & 2
    s = gpu["send_slot"]
    assert np.array_equal(np.sort(s[s >= 0]), np.arange(n - 37))


def test_notify_reads_any_nonzero_byte_as_true():
    x, idx, w = _random_case(300, 16, 64, 4, 4, 64, seed=6)
    import oracle
    in_rank = oracle.Oracle().layout(idx, 64, 16)["is_token_in_rank"] * np.uint8(7)
    gpu, ref = H.run_both(x, idx, w, 64, 16, 4, in_rank_override=in_rank)
    ref["is_token_in_rank"] = in_rank
    assert H.compare(gpu, ref) == []


def test_without_recv_topk_idx():
    x, idx, w = _random_case(300, 16, 64, 4, 4, 256, seed=8)
    gpu, ref = H.run_both(x, idx, w, 64, 16, 4, with_recv_idx=False)
    assert H.compare(gpu, ref) == []


def test_combine_flags_bad_send_slot():
    import torch

    from combine_ep_get_02_amd import ep

    rng = np.random.default_rng(2)
    T, R, K, Hd, n = 70, 8, 2, 64, 40
    slot = np.full((T, R), -1, np.int32)
    perm = rng.permutation(n)
    slot.reshape(-1)[rng.choice(T * R, n, replace=False)] = perm
    slot[3, 2] = n + 5   # out of range
    slot[9, 0] = -4      # below -1
    y = H.random_rows(rng, n, Hd)
    rw = rng.random((n, K)).astype(np.float32)
    import oracle
    ref = oracle.Oracle().combine(y, rw, slot, n)
    shape = ep.make_shape(T, Hd, K, 16, R, 4)
    out = torch.empty((T, Hd), dtype=torch.bfloat16, device="cuda")
    cw = torch.empty((T, K), dtype=torch.float32, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    ep.ep_combine(shape, H.to_dev_bf16(y), torch.from_numpy(rw).cuda(), torch.from_numpy(slot).cuda(), n, out, cw, st)
    torch.cuda.synchronize()
    assert np.array_equal(H.bf16_host(out), ref["combined_x"])
    assert np.array_equal(cw.cpu().numpy(), ref["combined_topk_weights"])
    assert int(st.item()) == 8 and ref["status"] == 8


# Combine of wide rows from 4096 tokens takes the staged form (consecutive tokens
# per block, rows written from LDS): 8 tokens a block for 14 KiB rows, 4 up to
# 28 KiB, 2 up to 56 KiB, the unstaged kernel beyond.  Ragged last blocks, rows
# that are not whole 2 KiB segments, tokens with no row and a bad slot.
STAGED = {
    # name: (T, R, K, H, fraction of (token, rank) pairs with a row)
    "eight_tokens_ragged_last_block": (4100, 8, 4, 7168, 0.5),
    "four_tokens_rows_897_units": (4099, 8, 2, 7176, 0.5),
    "four_tokens_20kib_rows": (4096, 8, 2, 10240, 0.4),
    "two_tokens_32kib_rows_one_token_last": (4097, 4, 2, 16384, 0.5),
    "two_tokens_56kib_rows": (4096, 2, 1, 28672, 0.5),
    "unstaged_64kib_rows": (4096, 2, 1, 32768, 0.5),
    "unstaged_below_4096_tokens": (4095, 8, 4, 7168, 0.5),
}


@pytest.mark.parametrize("name", sorted(STAGED))
def test_combine_staged_shapes(name):
    import torch

    import oracle
    from combine_ep_get_02_amd import ep

    T, R, K, Hd, frac = STAGED[name]
    print(f"[parity] combine staged shape={name}", flush=True)
    rng = np.random.default_rng(len(name) * 31 + T)
    have = rng.random((T, R)) < frac
    n = int(have.sum())
    slot = np.full((T, R), -1, np.int32)
    slot[have] = rng.permutation(n).astype(np.int32)
    slot[T - 1, R - 1] = n + 3  # out of range: flagged, the row skipped
    y = H.random_rows(rng, n, Hd)
    rw = rng.random((n, K)).astype(np.float32)
    ref = oracle.Oracle().combine(y, rw, slot, n)
    shape = ep.make_shape(T, Hd, K, 2 * R, R, 4)
    out = torch.empty((T, Hd), dtype=torch.bfloat16, device="cuda")
    out.view(torch.int16).fill_(-1)
    cw = torch.empty((T, K), dtype=torch.float32, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    ep.ep_combine(shape, H.to_dev_bf16(y), torch.from_numpy(rw).cuda(), torch.from_numpy(slot).cuda(), n, out, cw, st)
    torch.cuda.synchronize()
    assert np.array_equal(H.bf16_host(out), ref["combined_x"])
    assert np.array_equal(cw.cpu().numpy(), ref["combined_topk_weights"])
    assert int(st.item()) == ref["status"] == 8


# ---------------------------------------------------------------- fp8 rows and cached mode
def _fp8_case(x, idx, w, E, R, C, num_scales_block=128, capacity=None):
    """GPU: layout, notify, ep_dispatch_fp8, then ep_dispatch_cached of the same
    fp8 rows; oracle: the same stages.  Returns (gpu, ref) dicts."""
    import torch

    import oracle
    from combine_ep_get_02_amd import ep
    from combine_ep_get_02_amd.inputs import fp8_rows

    x8, sc = fp8_rows(x, num_scales_block) if num_scales_block else (x.view(np.uint8)[:, : x.shape[1]].copy(), None)
    T, H = x8.shape
    NS = 0 if sc is None else sc.shape[1]
    K = idx.shape[1]
    shape = ep.make_shape(T, H, K, E, R, C)
    cap = capacity if capacity is not None else T * min(R, K)
    b = ep.allocate(shape, 0)
    didx = torch.from_numpy(np.ascontiguousarray(idx)).cuda()
    dw = torch.from_numpy(np.ascontiguousarray(w)).cuda()
    ep.run_layout(b, didx)
    n = ep.run_notify(b, read_back=True)
    dx = torch.from_numpy(x8).cuda()
    dsc = torch.from_numpy(sc).cuda() if NS else None
    rx = torch.full((max(cap, 1), H), 0xAB, dtype=torch.uint8, device="cuda")
    rs = torch.full((max(cap, 1), max(NS, 1)), -2.0, dtype=torch.float32, device="cuda")
    rw = torch.full((max(cap, 1), K), -3.0, dtype=torch.float32, device="cuda")
    ri = torch.full((max(cap, 1), K), -777, dtype=torch.int64, device="cuda")
    si = torch.full((max(cap, 1), 2), -777, dtype=torch.int32, device="cuda")
    ss = torch.full((T, R), -777, dtype=torch.int32, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    ep.ep_dispatch_fp8(shape, dx, dsc, NS, didx, dw, b.in_rank, b.gbl, b.recv_gbl, b.workspace, cap, rx,
                       rs if NS else None, rw, ri, si,
                       ss, st)
    rows = min(n, cap)
    # cached mode: same rows again, into fresh buffers, from the recorded send_slot
    cx = torch.full((max(cap, 1), H), 0xCD, dtype=torch.uint8, device="cuda")
    cs = torch.full((max(cap, 1), max(NS, 1)), -4.0, dtype=torch.float32, device="cuda")
    ep.ep_dispatch_cached(shape, dx, 1, dsc, NS, ss, cap, cx, cs if NS else None, st)
    torch.cuda.synchronize()
    gpu = dict(send_slot=ss.cpu().numpy(), recv_x=rx[:rows].cpu().numpy(), recv_topk_weights=rw[:rows].cpu().numpy(),
               recv_topk_idx=ri[:rows].cpu().numpy(), recv_src_info=si[:rows].cpu().numpy(),
               cached_x=cx[:rows].cpu().numpy(), status=int(st.item()))
    if NS:
        gpu["recv_x_scales"] = rs[:rows].cpu().numpy()
        gpu["cached_scales"] = cs[:rows].cpu().numpy()
    o = oracle.Oracle()
    lay = o.layout(idx, E, R)
    note = o.notify(lay["is_token_in_rank"], lay["num_tokens_per_rank"], lay["num_tokens_per_rdma_rank"],
                    lay["num_tokens_per_expert"], C, 1)
    d = o.dispatch_fp8(x8, sc if NS else np.zeros((T, 0), np.float32), idx, w, lay["is_token_in_rank"],
                       note["gbl_channel_prefix_matrix"], note["recv_gbl_rank_prefix_sum"], E, recv_capacity=cap)
    c = o.dispatch_cached(x8, d["send_slot"], cap, sc if NS else None)
    ref = dict(send_slot=d["send_slot"], recv_x=d["recv_x"][:rows], recv_topk_weights=d["recv_topk_weights"][:rows],
               recv_topk_idx=d["recv_topk_idx"][:rows], recv_src_info=d["recv_src_info"][:rows],
               cached_x=c["recv_x"][:rows], status=d["status"] | c["status"])
    if NS:
        ref["recv_x_scales"] = d["recv_x_scales"][:rows]
        ref["cached_scales"] = c["recv_x_scales"][:rows]
    return gpu, ref


def _exact(gpu, ref):
    bad = []
    for k, r in ref.items():
        g = gpu[k]
        if k == "status":
            continue
        g, r = np.asarray(g), np.asarray(r)
        if g.shape != r.shape or not np.array_equal(g.view(np.uint8), r.view(np.uint8)):
            bad.append(k)
    return bad


@pytest.mark.parametrize("name", ["tiny", "sweep", "prefill", "skew", "large"])
def test_fp8_and_cached_dispatch_parity(name):
    print(f"[parity] fp8+cached workload={name}", flush=True)
    d = generate(name)
    wl = d["workload"]
    gpu, ref = _fp8_case(d["x"], d["topk_idx"], d["topk_weights"], wl.experts, wl.ranks, wl.channels)
    assert _exact(gpu, ref) == []
    assert gpu["status"] == 0 == ref["status"]


def test_fp8_many_scales_and_overflow():
    # 70 scales per token (more than one wave of lanes), and a receive capacity overflow
    x, idx, w = _random_case(300, 16, 64, 4, 5, 70 * 16, seed=12)
    import oracle
    n = int(oracle.Oracle().layout(idx, 64, 16)["num_tokens_per_rank"].sum())
    gpu, ref = _fp8_case(x, idx, w, 64, 16, 5, num_scales_block=16, capacity=n - 11)
    assert _exact(gpu, ref) == []
    assert gpu["status"] & 2 and ref["status"] & 2


def test_fp8_without_scales():
    x, idx, w = _random_case(200, 8, 32, 3, 4, 256, seed=13)
    gpu, ref = _fp8_case(x, idx, w, 32, 8, 4, num_scales_block=0)
    assert _exact(gpu, ref) == []


def test_cached_dispatch_bad_slots_bf16():
    import torch

    import oracle
    from combine_ep_get_02_amd import ep

    rng = np.random.default_rng(21)
    T, R, Hd, cap = 150, 16, 512, 600
    x = H.random_rows(rng, T, Hd)
    slot = np.full((T, R), -1, np.int32)
    picks = rng.choice(T * R, cap - 20, replace=False)
    slot.reshape(-1)[picks] = rng.permutation(cap)[: cap - 20]
    slot[4, 3] = cap + 9
    slot[7, 0] = -3
    shape = ep.make_shape(T, Hd, 2, 16, R, 4)
    out = torch.zeros((cap, Hd), dtype=torch.bfloat16, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    ep.ep_dispatch_cached(shape, H.to_dev_bf16(x), 2, None, 0, torch.from_numpy(slot).cuda(), cap, out, None, st)
    torch.cuda.synchronize()
    ref = oracle.Oracle().dispatch_cached(x, slot, cap)
    assert np.array_equal(H.bf16_host(out), ref["recv_x"])
    assert int(st.item()) == 8 and ref["status"] == 8


# cached mode at 2048 tokens and more: any slot map is copied exactly, out-of-range
# entries are flagged and skipped.  Maps: a random permutation of part of the capacity
# (no receive order at all), with bad entries; 16, 24 and 64 ranks, rows of 1 KiB to
# 16 KiB (some ragged), fp8 rows with 56 and 112 scales per token.
CACHED_LARGE = {
    # name: (T, R, row elements, element bytes, scales per token, capacity)
    "bf16_rows_897_units_r16": (2100, 16, 7176, 2, 0, 9000),
    "bf16_rows_16kib_r24": (2049, 24, 8192, 2, 0, 20000),
    "fp8_rows_14kib_r64_scales": (2304, 64, 14336, 1, 112, 12000),
    "bf16_rows_14kib_r64": (2048, 64, 7168, 2, 0, 15000),
    "bf16_rows_1kib_r24": (2049, 24, 512, 2, 0, 20000),
    "fp8_rows_7kib_scales": (2304, 64, 7168, 1, 56, 12000),
    "bf16_rows_14kib_r64_scales56": (2304, 64, 7168, 2, 56, 12000),
}


@pytest.mark.parametrize("form", [0, 1])  # EP_FORM_AUTO and EP_FORM_PUSH: cached mode's one (push) form
@pytest.mark.parametrize("name", sorted(CACHED_LARGE))
def test_cached_any_map_and_bad_slots(name, form):
    import torch

    import oracle
    from combine_ep_get_02_amd import ep

    T, R, Hd, elem, NS, cap = CACHED_LARGE[name]
    print(f"[parity] cached map={name}", flush=True)
    rng = np.random.default_rng(len(name) + 500)
    xr = rng.integers(0, 256, size=(T, Hd * elem), dtype=np.uint8)
    slot = np.full((T, R), -1, np.int32)
    picks = rng.choice(T * R, cap - 37, replace=False)
    slot.reshape(-1)[picks] = rng.permutation(cap)[: cap - 37]
    slot[5, R - 1] = cap + 9
    slot[T - 1, 0] = -3
    slot[1000, 2] = cap
    sc = rng.standard_normal((T, NS)).astype(np.float32) if NS else None
    shape = ep.make_shape(T, Hd, 2, 2 * R, R, 4)
    out = torch.full((cap, Hd * elem), 0x77, dtype=torch.uint8, device="cuda")
    outs = torch.full((cap, max(NS, 1)), -5.0, dtype=torch.float32, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    ep.ep_dispatch_cached(shape, torch.from_numpy(xr).cuda(), elem, torch.from_numpy(sc).cuda() if NS else None, NS,
                          torch.from_numpy(slot).cuda(), cap, out, outs if NS else None, st, form=form)
    torch.cuda.synchronize()
    # rows no entry names keep the fill, as in the oracle's output buffer below
    ref = oracle.Oracle().dispatch_cached(xr, slot, cap, sc)
    named = np.zeros(cap, bool)
    ok = (slot >= 0) & (slot < cap)
    named[slot[ok]] = True
    got = out.cpu().numpy()
    assert np.array_equal(got[named], ref["recv_x"][named])
    assert (got[~named] == 0x77).all()
    if NS:
        assert np.array_equal(outs.cpu().numpy()[named], ref["recv_x_scales"][named])
    assert int(st.item()) == 8 and ref["status"] == 8


def _group_case(x, idx, w, E, R, C, align, fp8=False, shrink=False, cap_delta=0, bad_ids=False, extra_rows=0,
                optional=True, extra_id=None):
    """Both sides run layout, notify, dispatch (bf16 or fp8 rows) and then the
    grouping by local expert, from the same inputs; the same host-side edits
    (a segment size shrunk, bad local ids, rows past the last slab) are made
    on both.  Returns (gpu, ref) dicts of the grouping outputs."""
    import torch

    import oracle
    from combine_ep_get_02_amd import ep
    from combine_ep_get_02_amd.inputs import fp8_rows

    T, K = idx.shape
    er = E // R
    xs, sc = (fp8_rows(x) if fp8 else (x, None))
    NS = 0 if sc is None else sc.shape[1]
    Hd = xs.shape[1]
    o = oracle.Oracle()
    lay = o.layout(idx, E, R)
    note = o.notify(lay["is_token_in_rank"], lay["num_tokens_per_rank"], lay["num_tokens_per_rdma_rank"],
                    lay["num_tokens_per_expert"], C, align)
    n = note["num_recv_tokens"]
    rows = n + extra_rows
    args = (idx, w, lay["is_token_in_rank"], note["gbl_channel_prefix_matrix"], note["recv_gbl_rank_prefix_sum"], E)
    d = o.dispatch_fp8(xs, sc, *args, recv_capacity=rows) if fp8 else o.dispatch(xs, *args, recv_capacity=rows)
    aligned = note["num_recv_tokens_per_expert"].astype(np.int32).copy()
    e_big = int(np.argmax(aligned)) if E else 0
    if shrink:
        aligned[e_big] -= align + 1
    r_idx, r_x = d["recv_topk_idx"].copy(), d["recv_x"].copy()
    r_w = d["recv_topk_weights"]
    slack_id = min(1, er - 1) if extra_id is None else extra_id
    if extra_rows:
        r_idx[n:] = slack_id
        r_x[n:] = 0
    if bad_ids and n > 1:
        r_idx[0, 0] = er + 3
        r_idx[min(5, n - 1), K - 1] = -5
    cap = max(int(np.maximum(aligned, 0).sum()) + cap_delta, 0)
    ref = o.group_by_expert(r_x, r_idx, r_w, note["recv_gbl_rank_prefix_sum"], aligned, E, grouped_capacity=cap,
                            recv_x_scales=d["recv_x_scales"] if fp8 else None)

    shape = ep.make_shape(T, x.shape[1], K, E, R, C, 0, align)
    b = ep.allocate(shape, rows)
    didx = torch.from_numpy(np.ascontiguousarray(idx)).cuda()
    dw = torch.from_numpy(np.ascontiguousarray(w)).cuda()
    ep.run_layout(b, didx)
    ep.run_notify(b)
    if fp8:
        rx = torch.zeros((max(rows, 1), Hd), dtype=torch.uint8, device="cuda")
        rs = torch.zeros((max(rows, 1), NS), dtype=torch.float32, device="cuda")
        ep.ep_dispatch_fp8(shape, torch.from_numpy(xs).cuda(), torch.from_numpy(sc).cuda(), NS, didx, dw, b.in_rank,
                           b.gbl, b.recv_gbl,
                           b.workspace, rows, rx, rs, b.recv_w, b.recv_idx, b.src_info, b.send_slot, b.dev_status)
    else:
        rx = b.recv_x
        rx[n:].zero_()
        rs = None
        ep.run_dispatch(b, torch.from_numpy(np.ascontiguousarray(xs).view(np.int16)).cuda().view(torch.bfloat16),
                        didx, dw)
    g_aligned = b.recv_per_expert.clone()
    if shrink:
        g_aligned[e_big] -= align + 1
    if extra_rows:
        b.recv_idx[n:] = slack_id
    if bad_ids and n > 1:
        b.recv_idx[0, 0] = er + 3
        b.recv_idx[min(5, n - 1), K - 1] = -5
    elem = 1 if fp8 else 2
    gx = torch.full((max(cap, 1), Hd * elem), 0x5A, dtype=torch.uint8, device="cuda")
    gs = torch.full((max(cap, 1), max(NS, 1)), -9.0, dtype=torch.float32, device="cuda")
    grow = torch.full((max(cap, 1),), -777, dtype=torch.int32, device="cuda")
    gw = torch.full((max(cap, 1),), -9.0, dtype=torch.float32, device="cuda")
    pos = torch.full((max(rows, 1), K), -777, dtype=torch.int32, device="cuda")
    m = torch.full((1,), -777, dtype=torch.int32, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    ep.ep_group_by_expert(shape, rx, elem, rs, NS, b.recv_idx, b.recv_w, b.recv_gbl, g_aligned, rows, cap, gx,
                          gs if NS else None, grow, gw if optional else None, pos if optional else None, m, st)
    torch.cuda.synchronize()
    mm = min(ref["num_grouped_rows"], cap)
    gpu = dict(num_grouped_rows=int(m.item()), grouped_x=gx[:mm].cpu().numpy().view(r_x.dtype),
               grouped_row=grow[:mm].cpu().numpy(), status=int(st.item()),
               untouched=bool((grow[mm:cap] == -777).all().item()) and bool((gx[mm:cap] == 0x5A).all().item()))
    want = dict(num_grouped_rows=ref["num_grouped_rows"], grouped_x=ref["grouped_x"][:mm],
                grouped_row=ref["grouped_row"][:mm], status=ref["status"], untouched=True)
    if optional:
        gpu["grouped_weights"] = gw[:mm].cpu().numpy()
        gpu["slot_pos"] = pos[:rows].cpu().numpy()
        want["grouped_weights"] = ref["grouped_weights"][:mm]
        want["slot_pos"] = ref["slot_pos"]
    if NS:
        gpu["grouped_x_scales"] = gs[:mm].cpu().numpy()
        want["grouped_x_scales"] = ref["grouped_x_scales"][:mm]
    return gpu, want


def _group_diff(gpu, want):
    bad = [k for k in ("num_grouped_rows", "status", "untouched") if gpu[k] != want[k]]
    return bad + _exact({k: v for k, v in gpu.items() if k not in bad},
                        {k: v for k, v in want.items() if k not in ("num_grouped_rows", "status", "untouched")})


@pytest.mark.parametrize("name,align", [("tiny", 4), ("sweep", 128), ("prefill", 1), ("skew", 4), ("large", 8)])
def test_group_by_expert_parity(name, align):
    print(f"[parity] group_by_expert workload={name} align={align}", flush=True)
    d = generate(name)
    wl = d["workload"]
    gpu, want = _group_case(d["x"], d["topk_idx"], d["topk_weights"], wl.experts, wl.ranks, wl.channels, align)
    assert _group_diff(gpu, want) == []
    assert want["status"] == 0


def test_group_fp8_rows_with_scales():
    print("[parity] group_by_expert fp8 rows, sweep", flush=True)
    d = generate("sweep")
    wl = d["workload"]
    gpu, want = _group_case(d["x"], d["topk_idx"], d["topk_weights"], wl.experts, wl.ranks, wl.channels, 2, fp8=True)
    assert _group_diff(gpu, want) == []


def test_group_overflow_bad_ids_and_rows_past_the_slabs():
    print("[parity] group_by_expert overflow / bad ids / extra rows", flush=True)
    x, idx, w = _random_case(600, 8, 64, 6, 5, 256, seed=31, mask_frac=0.1)
    gpu, want = _group_case(x, idx, w, 64, 8, 5, 4, shrink=True, cap_delta=-7, bad_ids=True, extra_rows=3)
    assert _group_diff(gpu, want) == []
    assert want["status"] == 3  # overflow and bad ids, both flagged


def test_group_512_local_experts_k32_duplicates():
    print("[parity] group_by_expert 512 local experts, k=32", flush=True)
    x, idx, w = _random_case(300, 2, 1024, 32, 3, 64, seed=32, mask_frac=0.2, dup=True)
    gpu, want = _group_case(x, idx, w, 1024, 2, 3, 2)
    assert _group_diff(gpu, want) == []


def test_group_without_optional_outputs():
    print("[parity] group_by_expert no weights / slot_pos", flush=True)
    d = generate("tiny")
    wl = d["workload"]
    gpu, want = _group_case(d["x"], d["topk_idx"], d["topk_weights"], wl.experts, wl.ranks, wl.channels, 3,
                            optional=False)
    assert _group_diff(gpu, want) == []


def test_group_no_rows():
    print("[parity] group_by_expert with no received rows", flush=True)
    x, idx, w = _random_case(40, 8, 16, 2, 4, 64, seed=33, mask_frac=1.0)
    gpu, want = _group_case(x, idx, w, 16, 8, 4, 4)
    assert _group_diff(gpu, want) == [] and gpu["num_grouped_rows"] == 0


def test_group_ignores_capacity_slack():
    # rows past the last slab (a capacity larger than N, as inside a captured graph) hold
    # out-of-range ids: not read, not flagged, their slot positions -1
    print("[parity] group_by_expert capacity slack", flush=True)
    x, idx, w = _random_case(500, 16, 64, 4, 7, 128, seed=34)
    gpu, want = _group_case(x, idx, w, 64, 16, 7, 2, extra_rows=37, extra_id=999)
    assert _group_diff(gpu, want) == []
    assert want["status"] == 0


def test_fp8_max_scales():
    # 1024 scales per token, the limit (16384 one-byte elements in 16-element blocks)
    print("[parity] fp8 with 1024 scales per token", flush=True)
    x, idx, w = _random_case(50, 8, 32, 4, 3, 16384, seed=14)
    gpu, ref = _fp8_case(x, idx, w, 32, 8, 3, num_scales_block=16)
    assert gpu["recv_x_scales"].shape[1] == 1024
    assert _exact(gpu, ref) == []
    assert gpu["status"] == 0 == ref["status"]


def test_combine_without_combined_weights():
    # combined_topk_weights is optional: the rows must not change and the buffer stays untouched
    print("[parity] combine without combined weights", flush=True)
    import torch

    from combine_ep_get_02_amd import ep

    d = generate("sweep")
    wl = d["workload"]
    gpu, ref = H.run_both(d["x"], d["topk_idx"], d["topk_weights"], wl.experts, wl.ranks, wl.channels)
    assert H.compare(gpu, ref) == []
    shape = ep.make_shape(wl.tokens, wl.hidden, wl.topk, wl.experts, wl.ranks, wl.channels)
    n = ref["num_recv_tokens"]
    b = ep.allocate(shape, n)
    didx = torch.from_numpy(d["topk_idx"]).cuda()
    ep.run_layout(b, didx)
    ep.run_notify(b)
    ep.run_dispatch(b, H.to_dev_bf16(d["x"]), didx, torch.from_numpy(d["topk_weights"]).cuda())
    b.combined_w.fill_(-5.0)
    ep.run_combine(b, with_weights=False)
    torch.cuda.synchronize()
    assert np.array_equal(H.bf16_host(b.combined_x), ref["combined_x"])
    assert bool((b.combined_w == -5.0).all().item())
    assert int(b.dev_status.item()) == 0


def test_every_call_without_a_status_word():
    # dev_status is optional in every entry point: same outputs with and without it,
    # on inputs that would set flags (bad ids, a short receive capacity)
    print("[parity] every entry point with dev_status = NULL", flush=True)
    import torch

    from combine_ep_get_02_amd import ep

    x, idx, w = _random_case(300, 16, 64, 4, 5, 128, seed=41)
    idx[3, 1] = 999  # a bad id: flagged when a status word is given
    shape = ep.make_shape(300, 128, 4, 64, 16, 5, 0, 2)
    didx, dw, dx = torch.from_numpy(idx).cuda(), torch.from_numpy(w).cuda(), H.to_dev_bf16(x)
    outs = []
    for with_status in (True, False):
        st = torch.zeros(1, dtype=torch.int32, device="cuda") if with_status else None
        b = ep.allocate(shape, 0)
        ep.ep_get_layout(shape, didx, b.per_rank, b.per_node, b.per_expert, b.in_rank, b.workspace, st)
        n = ep.ep_notify(shape, b.in_rank, b.per_rank, b.per_node, b.per_expert, b.gbl, b.rdma, b.recv_gbl,
                         b.recv_rdma, b.recv_per_expert, b.num_recv, b.workspace, True, st)
        cap = n - 5
        b2 = ep.allocate(shape, cap)
        ep.ep_get_layout(shape, didx, b2.per_rank, b2.per_node, b2.per_expert, b2.in_rank, b2.workspace, st)
        ep.ep_notify(shape, b2.in_rank, b2.per_rank, b2.per_node, b2.per_expert, b2.gbl, b2.rdma, b2.recv_gbl,
                     b2.recv_rdma, b2.recv_per_expert, b2.num_recv, b2.workspace, False, st)
        ep.ep_dispatch(shape, dx, didx, dw, b2.in_rank, b2.gbl, b2.recv_gbl, b2.workspace, cap, b2.recv_x, b2.recv_w,
                       b2.recv_idx,
                       b2.src_info, b2.send_slot, st)
        ep.ep_combine(shape, b2.recv_x, b2.recv_w, b2.send_slot, cap, b2.combined_x, b2.combined_w, st)
        m = int(b2.recv_per_expert.sum().item())
        g = ep.allocate_group(b2, m)
        ep.ep_group_by_expert(shape, b2.recv_x, 2, None, 0, b2.recv_idx, b2.recv_w, b2.recv_gbl, b2.recv_per_expert,
                              cap, m, g.grouped_x, None, g.grouped_row, g.grouped_w, g.slot_pos, g.num_grouped, st)
        torch.cuda.synchronize()
        mm = min(int(g.num_grouped.item()), m)
        outs.append([b2.send_slot.cpu(), b2.recv_x[:cap].view(torch.int16).cpu(), b2.combined_x.view(torch.int16).cpu(),
                     b2.combined_w.cpu(), g.grouped_row[:mm].cpu(), g.grouped_x[:mm].view(torch.int16).cpu()])
        if with_status:
            assert int(st.item()) & 3 == 3  # the bad id and the overflow were flagged
    assert all(torch.equal(a, b) for a, b in zip(*outs))


# ---- the pull form of dispatch (from 2048 tokens, rows of 1 KiB or more):
# ragged groups and chunks, ragged last tasks of a row, 1 / 3-node / 64 ranks,
# duplicates and masked slots, k = 32, and a receive capacity below N.
PULL = {
    # name: (T, R, E, K, C, H, extra)
    "groups_ragged_rows_513_units": (2100, 8, 64, 8, 6, 4104, {}),
    "rows_1kib_r24_masked": (2049, 24, 48, 4, 7, 512, dict(mask_frac=0.2)),
    "rows_7kib_r64_duplicates": (2304, 64, 256, 8, 24, 3584, dict(dup=True)),
    "single_rank": (2048, 1, 4, 2, 3, 1024, {}),
    "k32_r64": (2200, 64, 128, 32, 9, 2048, {}),
    "half_masked": (4096, 32, 256, 8, 24, 1024, dict(mask_frac=0.5)),
    "rows_16kib": (2048, 16, 64, 6, 5, 8192, {}),
}


@pytest.mark.parametrize("name", sorted(PULL))
def test_pull_dispatch_parity(name):
    T, R, E, K, C, H_, extra = PULL[name]
    print(f"[parity] pull={name}", flush=True)
    x, idx, w = _random_case(T, R, E, K, C, H_, seed=len(name) + 100, **extra)
    gpu, ref = H.run_both(x, idx, w, E, R, C)
    assert H.compare(gpu, ref) == []
    assert all(v == 0 for v in H.combine_bit_differences(gpu, ref).values())
    assert gpu["dev_status"] == ref["status"] == 0


def test_pull_dispatch_capacity_overflow():
    print("[parity] pull capacity overflow", flush=True)
    x, idx, w = _random_case(2100, 16, 64, 6, 5, 4104, seed=21)
    import oracle
    n = int(oracle.Oracle().layout(idx, 64, 16)["num_tokens_per_rank"].sum())
    gpu, ref = H.run_both(x, idx, w, 64, 16, 5, capacity=n - 1000)
    assert H.compare(gpu, ref) == []
    assert gpu["dev_status"] & 2 and ref["status"] & 2
    s = gpu["send_slot"]
    assert np.array_equal(np.sort(s[s >= 0]), np.arange(n - 1000))


def test_pull_fp8_ragged_groups_and_overflow():
    print("[parity] pull fp8", flush=True)
    x, idx, w = _random_case(2100, 64, 256, 8, 24, 7168, seed=22)
    import oracle
    n = int(oracle.Oracle().layout(idx, 256, 64)["num_tokens_per_rank"].sum())
    gpu, ref = _fp8_case(x, idx, w, 256, 64, 24)
    assert _exact(gpu, ref) == []
    assert gpu["status"] == 0 == ref["status"]
    gpu, ref = _fp8_case(x, idx, w, 256, 64, 24, capacity=n - 333)
    assert _exact(gpu, ref) == []
    assert gpu["status"] & 2 and ref["status"] & 2


# ---- dispatch straight into the grouped layout (ep_dispatch_grouped): every output
# equals the oracle's dispatch followed by its grouping with num_recv_rows = the
# receive capacity; no receive rows are written.
def _dispatch_grouped_case(x, idx, w, E, R, C, align, fp8=False, recv_delta=0, gcap_delta=0, scale_block=128):
    import torch

    import oracle
    from combine_ep_get_02_amd import ep
    from combine_ep_get_02_amd.inputs import fp8_rows

    T, K = idx.shape
    xs, sc = (fp8_rows(x, scale_block) if fp8 else (x, None))
    NS = 0 if sc is None else sc.shape[1]
    Hd = xs.shape[1]
    o = oracle.Oracle()
    lay = o.layout(idx, E, R)
    note = o.notify(lay["is_token_in_rank"], lay["num_tokens_per_rank"], lay["num_tokens_per_rdma_rank"],
                    lay["num_tokens_per_expert"], C, align)
    n = note["num_recv_tokens"]
    rcap = max(n + recv_delta, 0)
    args = (idx, w, lay["is_token_in_rank"], note["gbl_channel_prefix_matrix"], note["recv_gbl_rank_prefix_sum"], E)
    d = o.dispatch_fp8(xs, sc, *args, recv_capacity=rcap) if fp8 else o.dispatch(xs, *args, recv_capacity=rcap)
    aligned = note["num_recv_tokens_per_expert"]
    gcap = max(int(np.maximum(aligned, 0).sum()) + gcap_delta, 0)
    ref = o.group_by_expert(d["recv_x"], d["recv_topk_idx"], d["recv_topk_weights"], note["recv_gbl_rank_prefix_sum"],
                            aligned, E, grouped_capacity=gcap, recv_x_scales=d["recv_x_scales"] if fp8 else None,
                            num_recv_rows=rcap)

    shape = ep.make_shape(T, x.shape[1], K, E, R, C, 0, align)
    b = ep.allocate(shape, 0)
    didx = torch.from_numpy(np.ascontiguousarray(idx)).cuda()
    dw = torch.from_numpy(np.ascontiguousarray(w)).cuda()
    ep.run_layout(b, didx)
    ep.run_notify(b)
    rw = torch.full((max(rcap, 1), K), -3.0, dtype=torch.float32, device="cuda")
    ri = torch.full((max(rcap, 1), K), -777, dtype=torch.int64, device="cuda")
    si = torch.full((max(rcap, 1), 2), -777, dtype=torch.int32, device="cuda")
    ss = torch.full((T, R), -777, dtype=torch.int32, device="cuda")
    elem = 1 if fp8 else 2
    gx = torch.full((max(gcap, 1), Hd * elem), 0x5A, dtype=torch.uint8, device="cuda")
    gs = torch.full((max(gcap, 1), max(NS, 1)), -9.0, dtype=torch.float32, device="cuda")
    grow = torch.full((max(gcap, 1),), -777, dtype=torch.int32, device="cuda")
    gw = torch.full((max(gcap, 1),), -9.0, dtype=torch.float32, device="cuda")
    pos = torch.full((max(rcap, 1), K), -777, dtype=torch.int32, device="cuda")
    m = torch.full((1,), -777, dtype=torch.int32, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    dx = torch.from_numpy(np.ascontiguousarray(xs).view(np.int16 if not fp8 else np.uint8)).cuda()
    ep.ep_dispatch_grouped(shape, dx, elem, torch.from_numpy(sc).cuda() if NS else None, NS, didx, dw, b.in_rank,
                           b.gbl, b.recv_gbl,
                           b.recv_per_expert, b.workspace, rcap, rw, ri, si, ss, gcap, gx, gs if NS else None, grow, gw,
                           pos, m, st)
    torch.cuda.synchronize()
    rows = min(n, rcap)
    mm = min(ref["num_grouped_rows"], gcap)
    gpu = dict(num_grouped_rows=int(m.item()), grouped_x=gx[:mm].cpu().numpy().view(d["recv_x"].dtype),
               grouped_row=grow[:mm].cpu().numpy(), grouped_weights=gw[:mm].cpu().numpy(),
               slot_pos=pos[:rcap].cpu().numpy(), send_slot=ss.cpu().numpy(),
               recv_topk_weights=rw[:rows].cpu().numpy(), recv_topk_idx=ri[:rows].cpu().numpy(),
               recv_src_info=si[:rows].cpu().numpy(), status=int(st.item()),
               untouched=bool((grow[mm:gcap] == -777).all().item()) and bool((gx[mm:gcap] == 0x5A).all().item()))
    want = dict(num_grouped_rows=ref["num_grouped_rows"], grouped_x=ref["grouped_x"][:mm],
                grouped_row=ref["grouped_row"][:mm], grouped_weights=ref["grouped_weights"][:mm],
                slot_pos=ref["slot_pos"], send_slot=d["send_slot"], recv_topk_weights=d["recv_topk_weights"][:rows],
                recv_topk_idx=d["recv_topk_idx"][:rows], recv_src_info=d["recv_src_info"][:rows],
                status=d["status"] | ref["status"], untouched=True)
    if NS:
        gpu["grouped_x_scales"] = gs[:mm].cpu().numpy()
        want["grouped_x_scales"] = ref["grouped_x_scales"][:mm]
    return gpu, want


@pytest.mark.parametrize("name,align", [("tiny", 4), ("sweep", 128), ("prefill", 1), ("skew", 4), ("large", 8)])
def test_dispatch_grouped_parity(name, align):
    print(f"[parity] dispatch_grouped workload={name} align={align}", flush=True)
    d = generate(name)
    wl = d["workload"]
    gpu, want = _dispatch_grouped_case(d["x"], d["topk_idx"], d["topk_weights"], wl.experts, wl.ranks, wl.channels,
                                       align)
    assert _group_diff(gpu, want) == []
    assert gpu["status"] == 0


@pytest.mark.parametrize("name", ["sweep", "prefill", "skew"])
def test_dispatch_grouped_fp8_rows_with_scales(name):
    print(f"[parity] dispatch_grouped fp8 workload={name}", flush=True)
    d = generate(name)
    wl = d["workload"]
    gpu, want = _dispatch_grouped_case(d["x"], d["topk_idx"], d["topk_weights"], wl.experts, wl.ranks, wl.channels, 4,
                                       fp8=True)
    assert _group_diff(gpu, want) == []


def test_dispatch_grouped_short_capacities():
    # receive rows past a short receive capacity are dropped and not grouped; a short
    # grouped capacity drops the entries past it (both flagged)
    print("[parity] dispatch_grouped short capacities", flush=True)
    x, idx, w = _random_case(3000, 16, 64, 6, 5, 1000, seed=31, mask_frac=0.1, dup=True)
    for rd, gd in ((-700, 0), (0, -900), (-50, -50), (300, 0)):
        gpu, want = _dispatch_grouped_case(x, idx, w, 64, 16, 5, 4, recv_delta=rd, gcap_delta=gd)
        assert _group_diff(gpu, want) == [], (rd, gd)
        assert (gpu["status"] != 0) == (rd < 0 or gd < 0), (rd, gd, gpu["status"])


# the pull form of the rows straight from x (from 2048 tokens, rows of 1 KiB to 1 MiB,
# E <= 2048): ragged token groups and ragged row pieces, k = 32 with duplicates and
# masked slots, padding from expert_alignment, E at the limit and past it (push form)
GROUPED_PULL = {
    # name: (T, R, E, K, C, H, align, extra)
    "ragged_groups_rows_513_units": (2100, 8, 64, 8, 6, 4104, 4, {}),
    "k32_r64_duplicates_masked": (2200, 64, 128, 32, 9, 2048, 8, dict(dup=True, mask_frac=0.2)),
    "rows_1kib_r24_masked": (2049, 24, 48, 4, 7, 512, 1, dict(mask_frac=0.2)),
    "rows_16kib_k6": (2048, 16, 64, 6, 5, 8192, 3, {}),
    "e2048": (2048, 64, 2048, 8, 24, 1024, 2, {}),
    "e4096_push_form": (2048, 64, 4096, 8, 24, 512, 2, {}),
    # ~20 groups an XCD: the per-expert counts carried over many rounds
    "many_groups_t20000": (20000, 64, 256, 8, 24, 512, 4, dict(mask_frac=0.05)),
    # 16 slots a token: the ranking in two passes, the counts between groups after the copies
    "k16_many_groups": (9000, 32, 128, 16, 12, 512, 1, dict(dup=True)),
    # 512 experts (every wave scans the counts) and 640 (the block scan)
    "e512_wave_scan": (4100, 64, 512, 8, 24, 512, 1, {}),
    "e640_block_scan": (4100, 64, 640, 8, 24, 512, 1, {}),
}


@pytest.mark.parametrize("name", sorted(GROUPED_PULL))
def test_dispatch_grouped_pull_parity(name):
    T, R, E, K, C, H_, align, extra = GROUPED_PULL[name]
    print(f"[parity] dispatch_grouped pull={name}", flush=True)
    x, idx, w = _random_case(T, R, E, K, C, H_, seed=len(name) + 300, **extra)
    gpu, want = _dispatch_grouped_case(x, idx, w, E, R, C, align)
    assert _group_diff(gpu, want) == []
    assert gpu["status"] == 0


@pytest.mark.parametrize("H_", [7168, 1024])
def test_all_tokens_to_one_rank(H_):
    # the most skewed routing: every token's slots on the experts of rank 3, so one slab
    # holds every receive row and 63 are empty; the pull forms of dispatch (runs of
    # length 0 around the only one), combine and the one-launch grouped dispatch (every
    # group's entries in 8 segments, 128 a wave's worth of one id at most)
    print(f"[parity] all tokens to one rank h={H_}", flush=True)
    T, R, E, K, C, align = 4096, 64, 512, 8, 24, 4
    rng = np.random.default_rng(77 + H_)
    epr = E // R
    idx = (3 * epr + np.stack([rng.permutation(epr)[:K] for _ in range(T)])).astype(np.int64)
    w = rng.random((T, K)).astype(np.float32)
    x = H.random_rows(rng, T, H_)
    gpu, ref = H.run_both(x, idx, w, E, R, C)
    assert H.compare(gpu, ref) == []
    assert all(v == 0 for v in H.combine_bit_differences(gpu, ref).values())
    assert gpu["num_recv_tokens"] == T and gpu["dev_status"] == 0
    g, want = _dispatch_grouped_case(x, idx, w, E, R, C, align)
    assert _group_diff(g, want) == []
    assert g["status"] == 0


def test_dispatch_grouped_pull_fp8_112_scales():
    # more scales per token than lanes in a wave, ragged groups, alignment padding
    print("[parity] dispatch_grouped pull fp8 112 scales", flush=True)
    x, idx, w = _random_case(2100, 16, 64, 6, 5, 7168, seed=41, mask_frac=0.1)
    gpu, want = _dispatch_grouped_case(x, idx, w, 64, 16, 5, 4, fp8=True, scale_block=64)
    assert _group_diff(gpu, want) == []
    assert gpu["status"] == 0


def test_dispatch_grouped_pull_short_capacities():
    print("[parity] dispatch_grouped pull short capacities", flush=True)
    x, idx, w = _random_case(3000, 16, 64, 6, 5, 1024, seed=32, mask_frac=0.1, dup=True)
    for rd, gd in ((-700, 0), (0, -900), (-50, -50), (300, 0)):
        gpu, want = _dispatch_grouped_case(x, idx, w, 64, 16, 5, 4, recv_delta=rd, gcap_delta=gd)
        assert _group_diff(gpu, want) == [], (rd, gd)
        assert (gpu["status"] != 0) == (rd < 0 or gd < 0), (rd, gd, gpu["status"])


def test_dispatch_grouped_pull_edges():
    # the pull form with nothing to copy: every slot masked; no receive rows (every
    # grouped row is padding); no grouped rows (nothing written, overflow flagged)
    print("[parity] dispatch_grouped pull edges", flush=True)
    x, idx, w = _random_case(2048, 16, 64, 4, 5, 1024, seed=51, mask_frac=1.0)
    gpu, want = _dispatch_grouped_case(x, idx, w, 64, 16, 5, 4)
    assert _group_diff(gpu, want) == [] and gpu["num_grouped_rows"] == 0 and gpu["status"] == 0
    x, idx, w = _random_case(2048, 16, 64, 4, 5, 1024, seed=52)
    gpu, want = _dispatch_grouped_case(x, idx, w, 64, 16, 5, 4, recv_delta=-10 ** 6)
    assert _group_diff(gpu, want) == [] and gpu["num_grouped_rows"] > 0 and gpu["status"] == 2
    gpu, want = _dispatch_grouped_case(x, idx, w, 64, 16, 5, 4, gcap_delta=-10 ** 6)
    assert _group_diff(gpu, want) == [] and gpu["status"] == 2


@pytest.mark.parametrize("T", [2300, 900])
@pytest.mark.parametrize("what", ["stale_workspace", "gbl_entry", "recv_prefix"])
def test_dispatch_grouped_flags_inconsistent_routing(T, what):
    # the one-launch form (from 2048 tokens) and the four-launch form check the routing
    # inputs as ep_dispatch does: a workspace notify filled for another routing, or a
    # prefix that disagrees with is_token_in_rank, is flagged
    import torch

    import oracle
    from combine_ep_get_02_amd import ep

    print(f"[parity] dispatch_grouped inconsistent {what} T={T}", flush=True)
    R, E, K, C, Hd, align = 16, 64, 4, 10, 512, 4
    x, idx, w = _random_case(T, R, E, K, C, Hd, seed=T + len(what))
    o = oracle.Oracle()
    lay = o.layout(idx, E, R)
    note = o.notify(lay["is_token_in_rank"], lay["num_tokens_per_rank"], lay["num_tokens_per_rdma_rank"],
                    lay["num_tokens_per_expert"], C, align)
    gbl = note["gbl_channel_prefix_matrix"].copy()
    recv = note["recv_gbl_rank_prefix_sum"].copy()
    shape = ep.make_shape(T, Hd, K, E, R, C, 0, align)
    b = ep.allocate(shape, 0)
    ws_idx = idx.copy()
    if what == "stale_workspace":  # notify ran for a routing with one token sent elsewhere
        ws_idx[T // 2, 0] = (idx[T // 2, 0] + E // 2) % E
    elif what == "gbl_entry":
        gbl[3, 4] += 1
    else:
        recv[5:] += 2
    ep.run_layout(b, torch.from_numpy(ws_idx).cuda())
    ep.run_notify(b)
    n = note["num_recv_tokens"]
    rcap = n + 64
    aligned = note["num_recv_tokens_per_expert"]
    gcap = int(np.maximum(aligned, 0).sum())
    i32 = dict(dtype=torch.int32, device="cuda")
    rw = torch.empty((rcap, K), dtype=torch.float32, device="cuda")
    ri = torch.empty((rcap, K), dtype=torch.int64, device="cuda")
    si = torch.empty((rcap, 2), **i32)
    ss = torch.empty((T, R), **i32)
    gx = torch.empty((gcap, Hd), dtype=torch.int16, device="cuda")
    grow = torch.empty(gcap, **i32)
    gw = torch.empty(gcap, dtype=torch.float32, device="cuda")
    pos = torch.empty((rcap, K), **i32)
    m = torch.empty(1, **i32)
    st = torch.zeros(1, **i32)
    ep.ep_dispatch_grouped(shape, torch.from_numpy(x.view(np.int16)).cuda(), 2, None, 0, torch.from_numpy(idx).cuda(),
                           torch.from_numpy(w).cuda(), torch.from_numpy(lay["is_token_in_rank"]).cuda(),
                           torch.from_numpy(gbl).cuda(), torch.from_numpy(recv).cuda(),
                           torch.from_numpy(aligned).cuda(), b.workspace, rcap, rw, ri, si, ss, gcap, gx, None, grow, gw,
                           pos, m, st)
    torch.cuda.synchronize()
    want = ep.EP_DEV_STALE_WORKSPACE if what == "stale_workspace" else ep.EP_DEV_COUNT_MISMATCH
    assert int(st.item()) & want, int(st.item())


def test_dispatch_grouped_no_tokens():
    x, idx, w = _random_case(0, 16, 64, 4, 8, 64, seed=1)
    gpu, want = _dispatch_grouped_case(x, idx, w, 64, 16, 8, 4)
    assert _group_diff(gpu, want) == []
    assert gpu["num_grouped_rows"] == 0
