"""The whole step captured in a HIP graph (torch.cuda.graph over the library's
stream-ordered calls) and replayed: the library allocates nothing, records no
memset and needs no host synchronisation inside a step (notify without its
host read-back), so every call is capturable.  Each replay runs on new input
values written eagerly between replays, with synchronisations in between, and
must equal an eager run of the same step on those values bit for bit; the
dispatch straight into the grouped layout, captured in the same graph, must
give the same grouped rows as the eager dispatch and grouping."""
import numpy as np
import pytest
import torch

from combine_ep_get_02_amd import ep
from combine_ep_get_02_amd.inputs import generate

pytestmark = pytest.mark.gpu


def _eager_reference(shape, x, idx, w, cap, m):
    b = ep.allocate(shape, cap)
    g = ep.allocate_group(b, m)
    ep.run_layout(b, idx)
    ep.run_notify(b)
    ep.run_dispatch(b, x, idx, w)
    ep.run_combine(b)
    ep.run_group(b, g)
    torch.cuda.synchronize()
    return b, g


def _outputs(b, g):
    """the written part of every output: N receive rows, M grouped rows"""
    n, m = int(b.num_recv.item()), int(g.num_grouped.item())
    return {"N": torch.tensor(n), "M": torch.tensor(m), "send_slot": b.send_slot.clone(),
            "recv_x": b.recv_x[:n].view(torch.int16).clone(), "recv_w": b.recv_w[:n].clone(), "gbl": b.gbl.clone(),
            "combined_x": b.combined_x.view(torch.int16).clone(), "combined_w": b.combined_w.clone(),
            "grouped_x": g.grouped_x[:m].view(torch.int16).clone(), "grouped_row": g.grouped_row[:m].clone(),
            "status": b.dev_status.clone()}


@pytest.mark.parametrize("name", ["sweep", "skew"])
def test_step_in_a_graph_replays_exactly(name):
    print(f"[graph] workload={name}", flush=True)
    d = generate(name)
    wl = d["workload"]
    T, H, K, E, R, C = wl.tokens, wl.hidden, wl.topk, wl.experts, wl.ranks, wl.channels
    shape = ep.make_shape(T, H, K, E, R, C, 0, 4)
    x = torch.from_numpy(d["x"].view(np.int16)).cuda().view(torch.bfloat16)
    idx = torch.from_numpy(d["topk_idx"]).cuda()
    w = torch.from_numpy(d["topk_weights"]).cuda()
    cap = T * min(R, K)  # every routing of these tokens fits
    m = T * K * 4        # grouped rows: at most (slots + alignment padding per expert) fits this bound for align 4
    m = max(m, int(((torch.bincount(idx[idx >= 0], minlength=E) + 3) // 4 * 4).sum().item()))

    # buffers the graph reads and writes; the inputs are overwritten in place between replays
    gx, gidx, gw = x.clone(), idx.clone(), w.clone()
    b = ep.allocate(shape, cap)
    gb = ep.allocate_group(b, m)
    gf = ep.allocate_group(b, m)  # the dispatch straight into the grouped layout writes here
    # warm up on a side stream, as torch asks before capture
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ep.run_layout(b, gidx)
        ep.run_notify(b)
        ep.run_dispatch(b, gx, gidx, gw)
        ep.run_combine(b)
        ep.run_group(b, gb)
        ep.run_dispatch_grouped(b, gf, gx, gidx, gw)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ep.run_layout(b, gidx)
        ep.run_notify(b)
        ep.run_dispatch(b, gx, gidx, gw)
        ep.run_combine(b)
        ep.run_group(b, gb)
        ep.run_dispatch_grouped(b, gf, gx, gidx, gw)

    rng = np.random.default_rng(77)
    for replay in range(3):
        # new inputs, written eagerly: rows scaled, routing permuted across tokens
        perm = torch.from_numpy(rng.permutation(T)).cuda()
        gidx.copy_(idx[perm])
        gw.copy_(w[perm])
        gx.copy_((x.float() * float(replay + 1)).to(torch.bfloat16))
        b.dev_status.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = _outputs(b, gb)
        rb, rg = _eager_reference(shape, gx.clone(), gidx.clone(), gw.clone(), cap, m)
        want = _outputs(rb, rg)
        mm = int(want["M"].item())
        got["fused_grouped_x"] = gf.grouped_x[:mm].view(torch.int16).clone()
        got["fused_grouped_row"] = gf.grouped_row[:mm].clone()
        want["fused_grouped_x"], want["fused_grouped_row"] = want["grouped_x"], want["grouped_row"]
        bad = [k for k in want if not torch.equal(got[k], want[k])]
        assert not bad, f"replay {replay}: {bad}"
        assert int(got["status"].item()) == 0


def _fp8_calls(shape, b, x, idx, w, S, out):
    """layout, notify, the quantiser, the fp8 dispatch of its output, the quantising dispatch, the
    dequantiser of its rows and the cached quantising dispatch from its send_slot, all on torch's current
    stream into the buffers of `out`"""
    T, H = shape.num_tokens, shape.hidden
    cap = out["rx"].shape[0]
    ep.run_layout(b, idx)
    ep.run_notify(b)
    ep.ep_quantize_fp8(x, T, H, S, out["q"], out["qs"])
    ep.ep_dispatch_fp8(shape, out["q"], out["qs"], S, idx, w, b.in_rank, b.gbl, b.recv_gbl, b.workspace, cap,
                       out["rx"], out["rs"], b.recv_w, b.recv_idx, b.src_info, out["slot"], b.dev_status)
    ep.ep_dispatch_to_fp8(shape, x, S, idx, w, b.in_rank, b.gbl, b.recv_gbl, b.workspace, cap, out["tx"], out["ts"],
                          b.recv_w, b.recv_idx, b.src_info, out["tslot"], b.dev_status)
    ep.ep_dequantize_fp8(out["tx"], out["ts"], cap, H, S, out["back"])
    ep.ep_dispatch_cached_to_fp8(shape, x, S, out["tslot"], cap, out["cx"], out["cs"], b.dev_status)


def _fp8_buffers(T, H, S, R, cap):
    u8, f32, i32 = dict(dtype=torch.uint8, device="cuda"), dict(dtype=torch.float32, device="cuda"), \
        dict(dtype=torch.int32, device="cuda")
    return {"q": torch.zeros((T, H), **u8), "qs": torch.zeros((T, S), **f32), "rx": torch.zeros((cap, H), **u8),
            "rs": torch.zeros((cap, S), **f32), "slot": torch.zeros((T, R), **i32), "tx": torch.zeros((cap, H), **u8),
            "ts": torch.zeros((cap, S), **f32), "tslot": torch.zeros((T, R), **i32),
            "back": torch.zeros((cap, H), dtype=torch.bfloat16, device="cuda"), "cx": torch.zeros((cap, H), **u8),
            "cs": torch.zeros((cap, S), **f32)}


def test_fp8_path_in_a_graph_replays_exactly():
    """The quantiser, the fp8 dispatch of its output, the quantising dispatch, the dequantiser and the cached
    quantising dispatch, captured
    after layout and notify in one graph and replayed on new inputs: every replay equals an eager run."""
    print("[graph] fp8 path, workload=sweep", flush=True)
    d = generate("sweep")
    wl = d["workload"]
    T, H, K, E, R, C = wl.tokens, wl.hidden, wl.topk, wl.experts, wl.ranks, wl.channels
    S = H // 128
    shape = ep.make_shape(T, H, K, E, R, C)
    x = torch.from_numpy(d["x"].view(np.int16)).cuda().view(torch.bfloat16)
    idx = torch.from_numpy(d["topk_idx"]).cuda()
    w = torch.from_numpy(d["topk_weights"]).cuda()
    cap = T * min(R, K)
    gx, gidx, gw = x.clone(), idx.clone(), w.clone()
    b = ep.allocate(shape, cap)
    out = _fp8_buffers(T, H, S, R, cap)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _fp8_calls(shape, b, gx, gidx, gw, S, out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _fp8_calls(shape, b, gx, gidx, gw, S, out)
    rng = np.random.default_rng(78)
    for replay in range(3):
        perm = torch.from_numpy(rng.permutation(T)).cuda()
        gidx.copy_(idx[perm])
        gw.copy_(w[perm])
        gx.copy_((x.float() * float(2 * replay + 3)).to(torch.bfloat16))
        b.dev_status.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        rb = ep.allocate(shape, cap)
        ref = _fp8_buffers(T, H, S, R, cap)
        _fp8_calls(shape, rb, gx.clone(), gidx.clone(), gw.clone(), S, ref)
        torch.cuda.synchronize()
        n = int(rb.num_recv.item())
        bad = [k for k in ("q", "qs", "slot", "tslot") if not torch.equal(out[k], ref[k])]
        bad += [k for k in ("rx", "rs", "tx", "ts", "cx", "cs") if not torch.equal(out[k][:n], ref[k][:n])]
        if not torch.equal(out["back"][:n].view(torch.int16), ref["back"][:n].view(torch.int16)):
            bad.append("back")
        assert not bad, f"replay {replay}: {bad}"
        assert torch.equal(out["tx"][:n], out["rx"][:n]) and torch.equal(out["ts"][:n], out["rs"][:n])
        assert int(b.dev_status.item()) == 0
