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
