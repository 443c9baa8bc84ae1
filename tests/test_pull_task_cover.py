"""A host model of how the pull-form kernels hand out their row tasks.

dispatch_pull_kernel and group_pull_kernel share one enumeration: per token
group, the output is cut into tasks (a run of U 1 KiB pieces of one row, TPR
tasks per row); the XCD's W waves take tasks k = wx, wx + W, ...; a wave
resolves them 64 at a time (lane i takes the task base + i: its rank by a
binary search over the run starts, its token by a select-bit over the rank's
column, or its entry of the group's list) and then works through them in a
loop of nbatch readlanes.  The model below restates that arithmetic step by
step, in integers, and checks that it issues every (row, piece) of a group
exactly once and at the row the routing defines (the oracle's send_slot, or
the grouping's positions), on the benchmark's workloads.  A pass rules out the
task arithmetic as the cause of a lost or repeated piece: no task is skipped,
repeated or sent to another row by the enumeration or the routing."""
import numpy as np
import pytest

import oracle
from combine_ep_get_02_amd.inputs import generate

CHUNK = 64
XCDS = 8


def _nth_set_bit(x: int, n: int) -> int:
    pos = 0
    w = 32
    while w >= 1:
        c = bin(x & ((1 << w) - 1)).count("1")
        take = 1 if n >= c else 0
        n -= take * c
        x >>= take * w
        pos += take * w
        w >>= 1
    return pos


def _wave_tasks(wx: int, W: int, tasks: int):
    """The tasks one wave works through, batch by batch, as the kernels loop:
    for base = 0, 64, ... while wx + base*W < tasks: nbatch = min(64, ceil(...))
    readlanes of lanes j < nbatch, lane j holding task wx + (base + j)*W."""
    out = []
    base = 0
    while wx + base * W < tasks:
        nb = (tasks - wx - base * W + W - 1) // W
        nbatch = nb if nb < 64 else 64
        for j in range(nbatch):
            k = wx + (base + j) * W
            assert k < tasks  # lane j of the batch holds a valid task
            out.append(k)
        base += 64
    return out


def _route_rank(pex: np.ndarray, rr: int) -> int:
    """The kernels' binary search over the run starts (lane r holds pex[r],
    lanes past the ranks INT32_MAX): r = the last rank whose run starts at or
    before rr."""
    r = 0
    step = 32
    while step >= 1:
        cand = r + step
        if pex[cand] <= rr:
            r = cand
        step >>= 1
    return r


def _routing(name):
    d = generate(name, with_x=False)
    wl = d["workload"]
    o = oracle.Oracle()
    lay = o.layout(d["topk_idx"], wl.experts, wl.ranks)
    note = o.notify(lay["is_token_in_rank"], lay["num_tokens_per_rank"], lay["num_tokens_per_rdma_rank"],
                    lay["num_tokens_per_expert"], wl.channels, wl.expert_alignment)
    x = np.zeros((wl.tokens, 8), np.uint16)
    dis = o.dispatch(x, d["topk_idx"], d["topk_weights"], lay["is_token_in_rank"], note["gbl_channel_prefix_matrix"],
                     note["recv_gbl_rank_prefix_sum"], wl.experts)
    return d, wl, lay, note, dis


@pytest.mark.parametrize("name", ["prefill", "skew", "large"])
def test_dispatch_pull_tasks_cover_every_piece_once(name):
    """dispatch_pull_kernel: 2 chunks a group, U pieces a task, 512 waves per XCD."""
    d, wl, lay, note, dis = _routing(name)
    T, R = wl.tokens, wl.ranks
    row_units = wl.hidden * 2 // 16
    U = 1 if row_units >= 14 * CHUNK else 2 if row_units >= 7 * CHUNK else 8 if row_units > 4 * CHUNK else 4
    TPR = (row_units + U * CHUNK - 1) // (U * CHUNK)
    W, GT = 512, 2 * CHUNK
    in_rank = lay["is_token_in_rank"].astype(bool)
    slab0 = np.concatenate([[0], note["recv_gbl_rank_prefix_sum"][:-1]]).astype(np.int64)
    send_slot = dis["send_slot"]
    issued = {}
    before = np.zeros(R, np.int64)  # tokens before the group, per rank
    for g in range((T + GT - 1) // GT):
        blk = in_rank[g * GT:(g + 1) * GT]
        cols = [[sum(1 << l for l in range(CHUNK) if c * CHUNK + l < blk.shape[0] and blk[c * CHUNK + l, r])
                 for r in range(R)] for c in (0, 1)]
        n = blk.sum(0)
        s0 = slab0 + before
        pex = np.full(64, 2 ** 31 - 1, np.int64)
        pex[:R] = np.cumsum(np.concatenate([[0], n[:-1]]))
        tasks = int(n.sum()) * TPR
        for wx in range(W):
            for k in _wave_tasks(wx, W, tasks):
                rr, part = divmod(k, TPR)
                r = _route_rank(pex, rr)
                o = rr - pex[r]
                row = int(s0[r] + o)
                cc, c, oc = cols[0][r], 0, o
                if oc >= bin(cc).count("1"):  # the second chunk
                    oc -= bin(cc).count("1")
                    c, cc = 1, cols[1][r]
                assert oc < bin(cc).count("1")
                tok = g * GT + c * CHUNK + _nth_set_bit(cc, oc)
                assert send_slot[tok, r] == row, f"task {k} of group {g}: token {tok} rank {r} row {row}"
                key = (row, part)
                assert key not in issued
                issued[key] = tok
        before += n
    n_rows = note["num_recv_tokens"]
    assert len(issued) == n_rows * TPR
    assert sorted({row for row, _ in issued}) == list(range(n_rows))


@pytest.mark.parametrize("name,align", [("prefill", 4), ("skew", 1), ("large", 8)])
def test_group_pull_tasks_cover_every_piece_once(name, align):
    """group_pull_kernel: the group's entries in position order (the list the
    kernel builds in LDS), 16 waves a block, 32 blocks per XCD."""
    d, wl, lay, note, dis = _routing(name)
    T, K, E, R = wl.tokens, wl.topk, wl.experts, wl.ranks
    aligned = -(-lay["num_tokens_per_expert"] // align) * align
    o = oracle.Oracle()
    grp = o.group_by_expert(np.zeros((note["num_recv_tokens"], 8), np.uint16), dis["recv_topk_idx"],
                            dis["recv_topk_weights"], note["recv_gbl_rank_prefix_sum"], aligned, E)
    row_units = wl.hidden * 2 // 16
    U = 1 if row_units >= 14 * CHUNK else 2 if row_units >= 7 * CHUNK else 8 if row_units > 4 * CHUNK else 4
    TPR = (row_units + U * CHUNK - 1) // (U * CHUNK)
    W, GT = 32 * 16, 128
    slot_pos, src = grp["slot_pos"], dis["recv_src_info"]
    # grouped position of every (token, slot): through the token's receive rows
    tok_pos = np.full((T, K), -1, np.int64)
    for row in range(note["num_recv_tokens"]):
        for j in range(K):
            if slot_pos[row, j] >= 0:
                tok_pos[src[row, 1], j] = slot_pos[row, j]
    issued = {}
    for g in range((T + GT - 1) // GT):
        tp = tok_pos[g * GT:(g + 1) * GT]
        ent = [(pos, t) for t in range(tp.shape[0]) for pos in tp[t] if pos >= 0]
        ent.sort()  # the kernel's list: positions ascending (per expert run, runs in expert order)
        tasks = len(ent) * TPR
        for wx in range(W):
            for k in _wave_tasks(wx, W, tasks):
                e, part = divmod(k, TPR)
                pos, t = ent[e]
                key = (int(pos), part)
                assert key not in issued
                issued[key] = g * GT + t
    entries = grp["grouped_row"] >= 0
    assert len(issued) == int(entries.sum()) * TPR
    for pos in np.nonzero(entries)[0][:: max(1, entries.sum() // 2000)]:
        assert issued[(int(pos), 0)] == src[grp["grouped_row"][pos], 1]
