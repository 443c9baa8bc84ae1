"""Parity of the E4M3 quantiser and dequantiser (ep_quantize_fp8, ep_dequantize_fp8) with the
oracle, bit for bit, through the C ABI: every bf16 value of [-448, 448] at scale 1, groups of 16
to 1024 channels with ragged row counts and rows that are not a whole number of 1024 channels,
groups that are all zero, signed zeros, bf16 subnormals or span the whole exponent range, the
prefill size, and the chain quantise -> ep_dispatch_fp8 -> dequantise against the same chain in
the oracle."""
import zlib

import numpy as np
import pytest
import torch

import oracle
import pins
from combine_ep_get_02_amd import ep
from combine_ep_get_02_amd.inputs import generate
from gpu_harness import bf16_host, to_dev_bf16

pytestmark = pytest.mark.gpu


def _quant_gpu(x: np.ndarray, S: int):
    rows, H = x.shape
    dx = to_dev_bf16(x) if rows else torch.empty((0, H), dtype=torch.bfloat16, device="cuda")
    q = torch.full((max(rows, 1), H), 0xAB, dtype=torch.uint8, device="cuda")
    s = torch.full((max(rows, 1), S), -2.0, dtype=torch.float32, device="cuda")
    ep.ep_quantize_fp8(dx, rows, H, S, q, s)
    torch.cuda.synchronize()
    return q[:rows].cpu().numpy(), s[:rows].cpu().numpy(), q, s


def _dequant_gpu(codes: np.ndarray, scales: np.ndarray):
    rows, H = codes.shape
    dq = torch.from_numpy(np.ascontiguousarray(codes)).cuda()
    ds = torch.from_numpy(np.ascontiguousarray(scales, dtype=np.float32)).cuda()
    out = torch.full((max(rows, 1), H), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    ep.ep_dequantize_fp8(dq, ds, rows, H, scales.shape[1], out)
    torch.cuda.synchronize()
    return bf16_host(out[:rows])


def _same_codes(name, got, want):
    assert got.shape == want.shape, name
    bad = np.flatnonzero(got.reshape(-1) != want.reshape(-1))
    assert bad.size == 0, f"{name}: {bad.size} codes differ, first at {bad[:5].tolist()}: " \
                          f"{got.reshape(-1)[bad[:5]].tolist()} vs {want.reshape(-1)[bad[:5]].tolist()}"


def _same_scales(name, got, want):
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), \
        f"{name}: {int((got.view(np.uint32) != want.view(np.uint32)).sum())} scales differ"


def test_quantize_every_bf16_value_at_scale_one():
    """Each group of 128 starts with 448 (or ends with -448), so 448 / a = 1 and the kernel's
    conversion meets every bf16 value of [-448, 448] unscaled: this checks gfx950's conversion
    (nearest, ties to even, signed zero, subnormals) against the oracle's definition."""
    print("[quant] every bf16 value at scale 1", flush=True)
    o = oracle.Oracle()
    allbf = (np.arange(1 << 16, dtype=np.uint32) << 16).view(np.float32)
    vals = allbf[np.isfinite(allbf) & (np.abs(allbf) <= 448)]
    bits = (vals.view(np.uint32) >> 16).astype(np.uint16)
    per = 127
    groups = -(-bits.size // per)
    body = np.zeros(groups * per, np.uint16)
    body[: bits.size] = bits
    body = body.reshape(groups, per)
    head = np.full((groups, 1), 0x43E0, np.uint16)  # 448.0
    for lead, name in ((np.hstack([head, body]), "448 first"), (np.hstack([body, head | 0x8000]), "-448 last")):
        filler = np.zeros(((-groups) % 8, 128), np.uint16)  # whole rows of 1024: groups of 448, 0, 0, ...
        filler[:, 0] = 0x43E0
        x = np.vstack([lead, filler]).reshape(-1, 1024)
        S = x.shape[1] // 128
        gq, gs, _, _ = _quant_gpu(x, S)
        rq, rs = o.quantize_e4m3(x, S)
        _same_scales(name, gs, rs)
        assert np.all(gs == 1.0)
        _same_codes(name, gq, rq)


# (rows, hidden, num_scales): groups of 16 .. 1024 channels; rows not a whole number of 1024
# channels (48, 96, 896, 2560, 1536); row counts that leave a wave half used
QUANT_SHAPES = [(37, 48, 3), (5, 96, 3), (129, 896, 14), (33, 7168, 56), (17, 2560, 10), (9, 1536, 3),
                (3, 7168, 7), (1, 1024, 1), (64, 64, 1), (2, 16, 1)]


@pytest.mark.parametrize("rows,hidden,S", QUANT_SHAPES)
def test_quantize_groups_parity(rows, hidden, S):
    print(f"[quant] rows={rows} hidden={hidden} scales={S}", flush=True)
    rng = np.random.default_rng(1000 + rows * 7 + hidden)
    x = pins.quantize_groups(rng, rows, hidden, S)
    gq, gs, _, _ = _quant_gpu(x, S)
    rq, rs = oracle.Oracle().quantize_e4m3(x, S)
    _same_scales("scales", gs, rs)
    _same_codes("codes", gq, rq)


def test_quantize_leaves_rows_past_the_end_alone():
    """Rows past num_rows (and their scales) are not written."""
    print("[quant] rows past the end", flush=True)
    rng = np.random.default_rng(5)
    x = pins.quantize_groups(rng, 6, 896, 7)
    dx = to_dev_bf16(x)
    q = torch.full((8, 896), 0xAB, dtype=torch.uint8, device="cuda")
    s = torch.full((8, 7), -2.0, dtype=torch.float32, device="cuda")
    ep.ep_quantize_fp8(dx, 5, 896, 7, q, s)
    torch.cuda.synchronize()
    rq, rs = oracle.Oracle().quantize_e4m3(x[:5], 7)
    _same_codes("codes", q[:5].cpu().numpy(), rq)
    _same_scales("scales", s[:5].cpu().numpy(), rs)
    assert torch.all(q[5:] == 0xAB) and torch.all(s[5:] == -2.0)


def test_quantize_prefill_size():
    """The fp8 dispatch's workload: 4096 tokens of 7168 channels, 56 scales per token."""
    print("[quant] prefill 4096 x 7168 / 56", flush=True)
    x = generate("prefill")["x"]
    gq, gs, _, _ = _quant_gpu(x, 56)
    rq, rs = oracle.Oracle().quantize_e4m3(x, 56)
    _same_scales("scales", gs, rs)
    _same_codes("codes", gq, rq)


@pytest.mark.parametrize("rows,hidden,S", [(257, 256, 2), (3, 7168, 56), (40, 48, 3), (2, 1024, 1)])
def test_dequantize_parity(rows, hidden, S):
    """Every code pattern, with scales of every magnitude; E4M3 NaN patterns must give NaN."""
    print(f"[dequant] rows={rows} hidden={hidden} scales={S}", flush=True)
    rng = np.random.default_rng(77 + rows)
    codes = rng.integers(0, 256, size=(rows, hidden), dtype=np.uint8)
    codes.reshape(-1)[:256] = np.arange(256, dtype=np.uint8)[: min(256, codes.size)]
    scales = np.exp2(rng.uniform(-80, 80, size=(rows, S))).astype(np.float32)
    scales.reshape(-1)[:3] = np.array([1.0, 2.0 ** -7, 3.0], np.float32)[: min(3, scales.size)]
    got = _dequant_gpu(codes, scales)
    want = oracle.Oracle().dequantize_e4m3(codes, scales)
    nan = (codes & 0x7F) == 0x7F
    gnan = ((got & 0x7F80) == 0x7F80) & ((got & 0x7F) != 0)
    assert np.array_equal(gnan, nan), "NaN codes and NaN outputs differ"
    assert np.array_equal(got[~nan], want[~nan]), f"{int((got[~nan] != want[~nan]).sum())} values differ"


@pytest.mark.parametrize("name", ["sweep", "prefill"])
def test_quantize_dispatch_dequantize_chain(name):
    """x -> ep_quantize_fp8 -> ep_dispatch_fp8 -> ep_dequantize_fp8 on the received rows, against
    the oracle's quantiser, fp8 dispatch and dequantiser on the same inputs."""
    print(f"[quant] chain workload={name}", flush=True)
    d = generate(name)
    wl = d["workload"]
    x, idx, w = d["x"], d["topk_idx"], d["topk_weights"]
    T, H = x.shape
    S = H // 128
    K = idx.shape[1]
    E, R, C = wl.experts, wl.ranks, wl.channels
    shape = ep.make_shape(T, H, K, E, R, C)
    b = ep.allocate(shape, 0)
    didx = torch.from_numpy(np.ascontiguousarray(idx)).cuda()
    dw = torch.from_numpy(np.ascontiguousarray(w)).cuda()
    ep.run_layout(b, didx)
    n = ep.run_notify(b, read_back=True)
    _, _, dq, dsc = _quant_gpu(x, S)
    cap = T * min(R, K)
    rx = torch.full((cap, H), 0xAB, dtype=torch.uint8, device="cuda")
    rs = torch.full((cap, S), -2.0, dtype=torch.float32, device="cuda")
    rw = torch.empty((cap, K), dtype=torch.float32, device="cuda")
    si = torch.empty((cap, 2), dtype=torch.int32, device="cuda")
    ss = torch.empty((T, R), dtype=torch.int32, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    ep.ep_dispatch_fp8(shape, dq, dsc, S, didx, dw, b.in_rank, b.gbl, b.recv_gbl, b.workspace, cap, rx, rs, rw, None,
                       si, ss, st)
    out = torch.empty((max(n, 1), H), dtype=torch.bfloat16, device="cuda")
    ep.ep_dequantize_fp8(rx, rs, n, H, S, out)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    o = oracle.Oracle()
    q, s = o.quantize_e4m3(x, S)
    lay = o.layout(idx, E, R)
    note = o.notify(lay["is_token_in_rank"], lay["num_tokens_per_rank"], lay["num_tokens_per_rdma_rank"],
                    lay["num_tokens_per_expert"], C, 1)
    dd = o.dispatch_fp8(q, s, idx, w, lay["is_token_in_rank"], note["gbl_channel_prefix_matrix"],
                        note["recv_gbl_rank_prefix_sum"], E, recv_capacity=cap)
    assert n == note["num_recv_tokens"]
    _same_codes("recv_x", rx[:n].cpu().numpy(), dd["recv_x"][:n])
    _same_scales("recv_x_scales", rs[:n].cpu().numpy(), dd["recv_x_scales"][:n])
    back = o.dequantize_e4m3(dd["recv_x"][:n], dd["recv_x_scales"][:n])
    assert np.array_equal(bf16_host(out[:n]), back)


def _dispatch_to_fp8_case(x, idx, w, E, R, C, S, capacity=None, use_workspace=True):
    """GPU: layout, notify, then ep_dispatch_to_fp8; oracle: quantise, layout, notify, fp8 dispatch."""
    T, H = x.shape
    K = idx.shape[1]
    shape = ep.make_shape(T, H, K, E, R, C)
    cap = capacity if capacity is not None else T * min(R, K)
    b = ep.allocate(shape, 0)
    didx = torch.from_numpy(np.ascontiguousarray(idx)).cuda()
    dw = torch.from_numpy(np.ascontiguousarray(w)).cuda()
    ep.run_layout(b, didx)
    n = ep.run_notify(b, read_back=True)
    rows = min(n, cap)
    dx = to_dev_bf16(x)
    rx = torch.full((max(cap, 1), H), 0xAB, dtype=torch.uint8, device="cuda")
    rs = torch.full((max(cap, 1), S), -2.0, dtype=torch.float32, device="cuda")
    rw = torch.full((max(cap, 1), K), -3.0, dtype=torch.float32, device="cuda")
    ri = torch.full((max(cap, 1), K), -777, dtype=torch.int64, device="cuda")
    si = torch.full((max(cap, 1), 2), -777, dtype=torch.int32, device="cuda")
    ss = torch.full((T, R), -777, dtype=torch.int32, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    ep.ep_dispatch_to_fp8(shape, dx, S, didx, dw, b.in_rank, b.gbl, b.recv_gbl, b.workspace if use_workspace else None,
                          cap, rx, rs, rw, ri, si, ss, st)
    torch.cuda.synchronize()
    gpu = dict(send_slot=ss.cpu().numpy(), recv_x=rx[:rows].cpu().numpy(), recv_x_scales=rs[:rows].cpu().numpy(),
               recv_topk_weights=rw[:rows].cpu().numpy(), recv_topk_idx=ri[:rows].cpu().numpy(),
               recv_src_info=si[:rows].cpu().numpy(), status=int(st.item()))
    o = oracle.Oracle()
    q, s = o.quantize_e4m3(x, S)
    lay = o.layout(idx, E, R)
    note = o.notify(lay["is_token_in_rank"], lay["num_tokens_per_rank"], lay["num_tokens_per_rdma_rank"],
                    lay["num_tokens_per_expert"], C, 1)
    d = o.dispatch_fp8(q, s, idx, w, lay["is_token_in_rank"], note["gbl_channel_prefix_matrix"],
                       note["recv_gbl_rank_prefix_sum"], E, recv_capacity=cap)
    ref = dict(send_slot=d["send_slot"], recv_x=d["recv_x"][:rows], recv_x_scales=d["recv_x_scales"][:rows],
               recv_topk_weights=d["recv_topk_weights"][:rows], recv_topk_idx=d["recv_topk_idx"][:rows],
               recv_src_info=d["recv_src_info"][:rows], status=d["status"])
    return gpu, ref


def _assert_same(gpu, ref):
    bad = [k for k in ref if k != "status" and not np.array_equal(np.asarray(gpu[k]).view(np.uint8),
                                                                   np.asarray(ref[k]).view(np.uint8))]
    assert not bad, bad
    assert gpu["status"] == ref["status"], (gpu["status"], ref["status"])


@pytest.mark.parametrize("name", ["tiny", "sweep", "prefill", "skew", "large"])
def test_dispatch_to_fp8_workloads(name):
    """The five workloads at full size, groups of 128 channels (large: 4096 channels, 32 scales)."""
    print(f"[quant] dispatch_to_fp8 workload={name}", flush=True)
    d = generate(name)
    wl = d["workload"]
    gpu, ref = _dispatch_to_fp8_case(d["x"], d["topk_idx"], d["topk_weights"], wl.experts, wl.ranks, wl.channels,
                                     wl.hidden // 128)
    _assert_same(gpu, ref)


# (tokens, hidden, num_scales, ranks, experts, topk, channels, capacity delta, workspace): every tiling
# of the quantising push form (whole 7168-channel rows with the rank sweep from 4096 tokens, 4096-channel
# segments below, 1024-channel segments for other widths, ragged when the width is not a whole number of
# them), groups of 16 to 1024 channels, a receive capacity short of N, and no workspace
DISPATCH_TO_FP8 = {
    "h7168_t4100_ragged_groups_of_tokens": (4100, 7168, 56, 16, 64, 6, 20, 0, True),
    "h7168_t2304_segments": (2304, 7168, 7, 64, 256, 8, 24, 0, True),
    "h7168_t300_g16_no_ws": (300, 7168, 448, 8, 32, 4, 6, 0, False),
    "h896_g64_ragged_segment": (777, 896, 14, 24, 48, 5, 9, -40, True),
    "h2560_g256": (513, 2560, 10, 4, 16, 3, 4, 0, False),
    "h1024_g1024": (200, 1024, 1, 32, 64, 8, 3, -100, True),
    "h48_g16": (129, 48, 3, 2, 4, 2, 2, 0, True),
}


@pytest.mark.parametrize("case", sorted(DISPATCH_TO_FP8))
def test_dispatch_to_fp8_shapes(case):
    T, H, S, R, E, K, C, dcap, use_ws = DISPATCH_TO_FP8[case]
    print(f"[quant] dispatch_to_fp8 {case}", flush=True)
    rng = np.random.default_rng(zlib.crc32(case.encode()))
    x = pins.quantize_groups(rng, T, H, S)
    idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int64)
    idx[rng.random((T, K)) < 0.1] = -1
    w = rng.random((T, K)).astype(np.float32)
    n_ref = None
    cap = None
    if dcap:
        o = oracle.Oracle()
        lay = o.layout(idx, E, R)
        n_ref = int(lay["num_tokens_per_rank"].sum())
        cap = n_ref + dcap
    gpu, ref = _dispatch_to_fp8_case(x, idx, w, E, R, C, S, capacity=cap, use_workspace=use_ws)
    _assert_same(gpu, ref)
    if dcap < 0:
        assert gpu["status"] & ep.EP_DEV_RECV_OVERFLOW


def test_quantize_and_dequantize_past_the_grid_cap():
    """More units than the launch's 65,536 blocks cover at once (16,400 rows of 16,384 channels: 16.8M
    lanes' worth against 16.78M), so waves loop; rows are independent, so the oracle checks a sample of
    them (first, last and random rows, and every row the second pass of the loop reaches)."""
    print("[quant] 16400 x 16384 / 128 scales (grid-stride loop)", flush=True)
    rows, H, S = 16400, 16384, 128
    per_pass = 65536 * 4 * 64 * 16 // H  # rows the first pass of the loop covers
    assert rows > per_pass
    rng = np.random.default_rng(31)
    x = (rng.standard_normal((rows, H), dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    dx = to_dev_bf16(x)
    q = torch.empty((rows, H), dtype=torch.uint8, device="cuda")
    s = torch.empty((rows, S), dtype=torch.float32, device="cuda")
    ep.ep_quantize_fp8(dx, rows, H, S, q, s)
    back = torch.empty((rows, H), dtype=torch.bfloat16, device="cuda")
    ep.ep_dequantize_fp8(q, s, rows, H, S, back)
    torch.cuda.synchronize()
    del dx
    sample = np.unique(np.concatenate([np.arange(8), np.arange(per_pass - 4, rows),
                                       rng.choice(rows, 64, replace=False)]))
    ts = torch.from_numpy(sample).cuda()
    gq, gs, gb = q[ts].cpu().numpy(), s[ts].cpu().numpy(), bf16_host(back[ts])
    o = oracle.Oracle()
    rq, rs = o.quantize_e4m3(x[sample], S)
    _same_scales("scales", gs, rs)
    _same_codes("codes", gq, rq)
    assert np.array_equal(gb, o.dequantize_e4m3(rq, rs))


QUANT_RANDOM_CASES = 10


def draw_quant(case: int) -> dict:
    """A seeded random configuration of the quantising dispatch: token counts around the chunk and
    128-token group boundaries and across the 4096-token tiling switch, 1 to 64 ranks, groups of 16
    to 1024 channels (every fourth case 7168 channels in 56 groups, the whole-row tilings), masked and
    duplicate ids, a capacity a few rows short, with or without the workspace."""
    rng = np.random.default_rng(7000 + case)
    R = int(rng.choice([1, 2, 4, 8, 16, 24, 32, 64]))
    E = R * int(rng.choice([1, 2, 4, 8, 16]))
    K = int(rng.integers(1, min(8, E) + 1))
    T = int(rng.choice([1, 63, 65, 333, 1000, 2049, 4096, 4100, 5000]))
    C = int(rng.integers(1, 50))
    if case % 4 == 0:
        g, S = 128, 56
    else:
        g = int(rng.choice([16, 32, 64, 128, 256, 512, 1024]))
        S = int(rng.integers(1, max(1, min(64, 8192 // g)) + 1))
    return dict(T=T, R=R, E=E, K=K, C=C, H=g * S, S=S, mask=float(rng.choice([0.0, 0.1, 0.4])),
                dup=bool(case % 3 == 1), short=bool(case % 4 == 2),
                ws=bool(case % 2 == 0) or -(-T // C) > 4096)


@pytest.mark.parametrize("case", range(QUANT_RANDOM_CASES))
def test_dispatch_to_fp8_random_shapes(case):
    c = draw_quant(case)
    print(f"[quant] dispatch_to_fp8 random case {case}: {c}", flush=True)
    rng = np.random.default_rng(8000 + case)
    T, R, E, K = c["T"], c["R"], c["E"], c["K"]
    idx = np.stack([rng.choice(E, K, replace=c["dup"]) for _ in range(T)]).astype(np.int64)
    if c["mask"]:
        flat = rng.choice(T * K, int(c["mask"] * T * K), replace=False)
        idx.reshape(-1)[flat] = -1
    w = rng.random((T, K)).astype(np.float32)
    x = pins.quantize_groups(rng, T, c["H"], c["S"])
    cap = None
    if c["short"]:
        n = int(oracle.Oracle().layout(idx, E, R)["num_tokens_per_rank"].sum())
        cap = max(0, n - 5)
    gpu, ref = _dispatch_to_fp8_case(x, idx, w, E, R, c["C"], c["S"], capacity=cap, use_workspace=c["ws"])
    _assert_same(gpu, ref)


@pytest.mark.parametrize("name", ["sweep", "prefill", "large"])
def test_dispatch_cached_to_fp8_replays_the_layout(name):
    """ep_dispatch_cached_to_fp8 with the send_slot ep_dispatch_to_fp8 wrote: the same codes and scales at
    the same rows, and the oracle's quantiser then cached dispatch bit for bit."""
    print(f"[quant] dispatch_cached_to_fp8 workload={name}", flush=True)
    d = generate(name)
    wl = d["workload"]
    x, idx, w = d["x"], d["topk_idx"], d["topk_weights"]
    T, H = x.shape
    K, S = idx.shape[1], H // 128
    shape = ep.make_shape(T, H, K, wl.experts, wl.ranks, wl.channels)
    b = ep.allocate(shape, 0)
    didx = torch.from_numpy(np.ascontiguousarray(idx)).cuda()
    dw = torch.from_numpy(np.ascontiguousarray(w)).cuda()
    ep.run_layout(b, didx)
    n = ep.run_notify(b, read_back=True)
    dx = to_dev_bf16(x)
    rx = torch.empty((n, H), dtype=torch.uint8, device="cuda")
    rs = torch.empty((n, S), dtype=torch.float32, device="cuda")
    rw = torch.empty((n, K), dtype=torch.float32, device="cuda")
    si = torch.empty((n, 2), dtype=torch.int32, device="cuda")
    ss = torch.empty((T, wl.ranks), dtype=torch.int32, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    ep.ep_dispatch_to_fp8(shape, dx, S, didx, dw, b.in_rank, b.gbl, b.recv_gbl, b.workspace, n, rx, rs, rw, None, si,
                          ss, st)
    cx = torch.full((n, H), 0x5A, dtype=torch.uint8, device="cuda")
    cs = torch.full((n, S), -4.0, dtype=torch.float32, device="cuda")
    ep.ep_dispatch_cached_to_fp8(shape, dx, S, ss, n, cx, cs, st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert torch.equal(cx, rx) and torch.equal(cs, rs)
    o = oracle.Oracle()
    q, s = o.quantize_e4m3(x, S)
    ref = o.dispatch_cached(q, ss.cpu().numpy(), n, s)
    _same_codes("recv_x", cx.cpu().numpy(), ref["recv_x"])
    _same_scales("recv_x_scales", cs.cpu().numpy(), ref["recv_x_scales"])


# (tokens, ranks, hidden, num_scales, capacity): whole 7168-channel rows from 4096 tokens, 4096-channel
# segments below, and 896-channel rows (1024-channel segments, ragged)
CACHED_QUANT = {"t4100_r16_h7168": (4100, 16, 7168, 56, 30000), "t2304_r64_h7168_g16": (2304, 64, 7168, 448, 12000),
                "t777_r24_h896_g64": (777, 24, 896, 14, 9000)}


@pytest.mark.parametrize("case", sorted(CACHED_QUANT))
def test_dispatch_cached_to_fp8_any_map_and_bad_slots(case):
    """A random injective map over part of the capacity with entries past it and below -1: named rows get
    the oracle's codes and scales, bad entries are skipped and flagged, other rows keep their contents."""
    T, R, H, S, cap = CACHED_QUANT[case]
    print(f"[quant] dispatch_cached_to_fp8 map={case}", flush=True)
    rng = np.random.default_rng(zlib.crc32(case.encode()))
    x = pins.quantize_groups(rng, T, H, S)
    slot = np.full((T, R), -1, np.int32)
    picks = rng.choice(T * R, cap - 41, replace=False)
    slot.reshape(-1)[picks] = rng.permutation(cap)[: cap - 41]
    slot[3, R - 1] = cap + 5
    slot[T - 1, 0] = -2
    slot[T // 2, 1 % R] = cap
    shape = ep.make_shape(T, H, 2, 2 * R, R, 4)
    out = torch.full((cap, H), 0x77, dtype=torch.uint8, device="cuda")
    outs = torch.full((cap, S), -5.0, dtype=torch.float32, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    ep.ep_dispatch_cached_to_fp8(shape, to_dev_bf16(x), S, torch.from_numpy(slot).cuda(), cap, out, outs, st)
    torch.cuda.synchronize()
    o = oracle.Oracle()
    q, s = o.quantize_e4m3(x, S)
    ref = o.dispatch_cached(q, slot, cap, s)
    named = np.zeros(cap, bool)
    ok = (slot >= 0) & (slot < cap)
    named[slot[ok]] = True
    got, gots = out.cpu().numpy(), outs.cpu().numpy()
    _same_codes("recv_x", got[named], ref["recv_x"][named])
    _same_scales("recv_x_scales", gots[named], ref["recv_x_scales"][named])
    assert (got[~named] == 0x77).all() and (gots[~named] == -5.0).all()
    assert int(st.item()) == ep.EP_DEV_BAD_SEND_SLOT and ref["status"] == ep.EP_DEV_BAD_SEND_SLOT


def test_quantising_dispatches_with_no_receive_capacity():
    """Capacity 0: every routed (token, rank) is dropped and flagged, send_slot is -1 throughout, nothing
    is stored (the oracle agrees); the cached form with a map of only -1 entries stores nothing either."""
    print("[quant] dispatch_to_fp8 with capacity 0", flush=True)
    rng = np.random.default_rng(90)
    T, H, S, R, E, K, C = 300, 896, 14, 16, 64, 4, 5
    idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int64)
    w = rng.random((T, K)).astype(np.float32)
    x = pins.quantize_groups(rng, T, H, S)
    gpu, ref = _dispatch_to_fp8_case(x, idx, w, E, R, C, S, capacity=0)
    _assert_same(gpu, ref)
    assert gpu["status"] == ep.EP_DEV_RECV_OVERFLOW and (gpu["send_slot"] == -1).all()
    shape = ep.make_shape(T, H, K, E, R, C)
    out = torch.full((4, H), 0x77, dtype=torch.uint8, device="cuda")
    outs = torch.full((4, S), -5.0, dtype=torch.float32, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    none = torch.full((T, R), -1, dtype=torch.int32, device="cuda")
    ep.ep_dispatch_cached_to_fp8(shape, to_dev_bf16(x), S, none, 4, out, outs, st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0 and (out == 0x77).all() and (outs == -5.0).all()


@pytest.mark.parametrize("case", range(8))
def test_quantize_dequantize_random_shapes(case):
    """Seeded random shapes for the quantiser and the dequantiser: 1 to 3000 rows, groups of 16 to 1024
    channels, 1 to 64 groups a row (rows up to 16384 channels), bit for bit against the oracle both ways."""
    rng = np.random.default_rng(9000 + case)
    g = int(rng.choice([16, 32, 64, 128, 256, 512, 1024]))
    S = int(rng.integers(1, min(64, 16384 // g) + 1))
    rows = int(rng.choice([1, 2, 7, 63, 64, 65, 500, 3000]))
    print(f"[quant] random case {case}: rows={rows} hidden={g * S} groups of {g}", flush=True)
    x = pins.quantize_groups(rng, rows, g * S, S)
    gq, gs, dq, ds = _quant_gpu(x, S)
    o = oracle.Oracle()
    rq, rs = o.quantize_e4m3(x, S)
    _same_scales("scales", gs, rs)
    _same_codes("codes", gq, rq)
    back = torch.empty((rows, g * S), dtype=torch.bfloat16, device="cuda")
    ep.ep_dequantize_fp8(dq, ds, rows, g * S, S, back)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_host(back), o.dequantize_e4m3(rq, rs))
