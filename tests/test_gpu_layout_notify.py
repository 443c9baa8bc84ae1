"""ep_layout_notify (layout and notify in one launch) against the two calls and the oracle.

Every output of ep_get_layout and ep_notify must come out of the fused call bit
for bit, on the five workloads at full size and on edge shapes (no tokens, fewer
tokens than channels, one rank, three nodes, experts past the LDS histogram,
enough chunks that the scan runs in global memory, masked and duplicate and
out-of-range ids, alignment).  The workspace it leaves must drive ep_dispatch
(the workspace path) to the oracle's rows, and a dirty completion ticket or
report word must be flagged."""
import numpy as np
import pytest
import torch

import gpu_harness as H
import oracle
from combine_ep_get_02_amd import ep
from combine_ep_get_02_amd.inputs import WORKLOADS, generate

pytestmark = pytest.mark.gpu

LAYOUT_KEYS = ("per_rank", "per_node", "per_expert", "in_rank")
NOTIFY_KEYS = ("gbl", "rdma", "recv_gbl", "recv_rdma", "recv_per_expert", "num_recv")
TICKET_FUSED = 32  # uint32 word of the workspace: the fused call's ticket (count), its report at word 34


def _case(T, R, E, K, seed, mask_frac=0.0, dup=False, bad=False):
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.choice(E, K, replace=dup) for _ in range(T)]).astype(np.int64) if T else \
        np.zeros((0, K), np.int64)
    if mask_frac and T:
        idx.reshape(-1)[rng.choice(T * K, int(mask_frac * T * K), replace=False)] = -1
    if bad and T > 10:
        idx[3, 0] = E + 5
        idx[7, K - 1] = -4
    return idx


def _both(idx, E, R, C, align=1):
    T, K = idx.shape
    shape = ep.make_shape(T, 64, K, E, R, C, 0, align)
    didx = torch.from_numpy(idx).cuda()
    a = ep.allocate(shape, 0)
    ep.run_layout(a, didx)
    n_a = ep.run_notify(a, read_back=True)
    b = ep.allocate(shape, 0)
    for t in (b.per_rank, b.per_node, b.per_expert, b.gbl, b.rdma, b.recv_gbl, b.recv_rdma, b.recv_per_expert,
              b.num_recv):
        t.fill_(-777)
    b.in_rank.fill_(0x5A)
    n_b = ep.run_layout_notify(b, didx, read_back=True)
    torch.cuda.synchronize()
    return a, b, n_a, n_b


def _check(idx, E, R, C, align=1):
    a, b, n_a, n_b = _both(idx, E, R, C, align)
    assert n_a == n_b
    for k in LAYOUT_KEYS + NOTIFY_KEYS:
        assert torch.equal(getattr(a, k), getattr(b, k)), k
    assert int(a.dev_status.item()) == int(b.dev_status.item())
    orc = oracle.Oracle()
    lay = orc.layout(idx, E, R)
    note = orc.notify(lay["is_token_in_rank"], lay["num_tokens_per_rank"], lay["num_tokens_per_rdma_rank"],
                      lay["num_tokens_per_expert"], C, align)
    assert np.array_equal(b.per_expert.cpu().numpy(), lay["num_tokens_per_expert"])
    assert np.array_equal(b.in_rank.cpu().numpy(), lay["is_token_in_rank"])
    assert np.array_equal(b.gbl.cpu().numpy(), note["gbl_channel_prefix_matrix"])
    assert np.array_equal(b.recv_per_expert.cpu().numpy(), note["num_recv_tokens_per_expert"])
    assert n_b == note["num_recv_tokens"]
    return a, b


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_fused_matches_two_calls_on_workloads(name):
    print(f"[layout+notify] workload={name}", flush=True)
    d = generate(name, with_x=False)
    wl = d["workload"]
    _check(d["topk_idx"], wl.experts, wl.ranks, wl.channels, wl.expert_alignment)


EDGES = {
    # name: (T, R, E, K, C, align, extra)
    "no_tokens": (0, 16, 64, 4, 8, 1, {}),
    "fewer_tokens_than_channels": (3, 8, 16, 2, 7, 1, {}),
    "one_block": (200, 16, 64, 6, 12, 4, {}),
    "few_blocks": (1000, 16, 64, 6, 12, 4, {}),
    "one_block_k_odd": (256, 8, 40, 5, 3, 1, dict(mask_frac=0.1, bad=True)),
    "one_rank": (1500, 1, 4, 2, 3, 1, {}),
    "three_nodes": (2100, 24, 48, 4, 6, 1, dict(mask_frac=0.2, dup=True)),
    "experts_past_lds": (3000, 64, 16384, 8, 24, 1, {}),
    "experts_past_lds_one_block": (250, 64, 16384, 8, 24, 1, {}),
    "experts_past_lds_few_blocks": (700, 64, 16384, 8, 24, 1, {}),
    "global_scan": (100000, 64, 256, 8, 24, 1, {}),
    "four_groups_a_lane": (40000, 64, 256, 8, 24, 1, {}),
    "just_past_64_groups": (16400, 16, 64, 6, 32, 1, {}),
    "many_channels": (5000, 16, 64, 4, 4096, 1, {}),
    "k32_bad_ids": (4100, 64, 128, 32, 9, 128, dict(dup=True, bad=True)),
    "five_ranks": (2000, 5, 10, 3, 4, 1, dict(mask_frac=1.0)),
}


@pytest.mark.parametrize("name", sorted(EDGES))
def test_fused_matches_two_calls_on_edges(name):
    T, R, E, K, C, align, extra = EDGES[name]
    print(f"[layout+notify] edge={name}", flush=True)
    _check(_case(T, R, E, K, seed=len(name) + T, **extra), E, R, C, align)


@pytest.mark.parametrize("name", ["prefill", "sweep"])
def test_fused_workspace_drives_dispatch(name):
    # the workspace the fused call leaves is notify's: dispatch's workspace path uses it
    print(f"[layout+notify] dispatch after fused, workload={name}", flush=True)
    d = generate(name)
    wl = d["workload"]
    T, K = d["topk_idx"].shape
    shape = ep.make_shape(T, wl.hidden, K, wl.experts, wl.ranks, wl.channels)
    didx = torch.from_numpy(d["topk_idx"]).cuda()
    b = ep.allocate(shape, 0)
    n = ep.run_layout_notify(b, didx, read_back=True)
    b2 = ep.allocate(shape, n)
    ep.run_layout_notify(b2, didx)
    b2.recv_x.view(torch.int16).fill_(-1)
    ep.run_dispatch(b2, H.to_dev_bf16(d["x"]), didx, torch.from_numpy(d["topk_weights"]).cuda())
    torch.cuda.synchronize()
    orc = oracle.Oracle()
    lay = orc.layout(d["topk_idx"], wl.experts, wl.ranks)
    note = orc.notify(lay["is_token_in_rank"], lay["num_tokens_per_rank"], lay["num_tokens_per_rdma_rank"],
                      lay["num_tokens_per_expert"], wl.channels)
    dis = orc.dispatch(d["x"], d["topk_idx"], d["topk_weights"], lay["is_token_in_rank"],
                       note["gbl_channel_prefix_matrix"], note["recv_gbl_rank_prefix_sum"], wl.experts)
    assert np.array_equal(b2.send_slot.cpu().numpy(), dis["send_slot"])
    assert np.array_equal(H.bf16_host(b2.recv_x), dis["recv_x"])
    assert np.array_equal(b2.recv_w.cpu().numpy(), dis["recv_topk_weights"])
    assert int(b2.dev_status.item()) == 0


@pytest.mark.parametrize("word,value", [(TICKET_FUSED, 1), (TICKET_FUSED, 16), (TICKET_FUSED + 2, 5)])
def test_fused_dirty_workspace_is_flagged(word, value):
    print(f"[layout+notify] dirty word={word} value={value}", flush=True)
    idx = _case(8192, 64, 256, 8, seed=2)
    shape = ep.make_shape(8192, 64, 8, 256, 64, 24)
    didx = torch.from_numpy(idx).cuda()
    b = ep.allocate(shape, 0)
    ep.run_layout_notify(b, didx)
    torch.cuda.synchronize()
    assert int(b.dev_status.item()) == 0
    gbl = b.gbl.clone()
    b.workspace.view(torch.int32)[word] = value
    ep.run_layout_notify(b, didx)
    torch.cuda.synchronize()
    assert int(b.dev_status.item()) & ep.EP_DEV_STALE_WORKSPACE
    b.workspace.zero_()
    b.dev_status.zero_()
    ep.run_layout_notify(b, didx)
    torch.cuda.synchronize()
    assert int(b.dev_status.item()) == 0 and torch.equal(b.gbl, gbl)
