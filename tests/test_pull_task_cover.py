"""A host model of how the pull-form kernels hand out their row tasks.

dispatch_pull_kernel and dispatch_grouped_pull_kernel share one enumeration: per
token group, the output is cut into tasks (a run of U 1 KiB pieces of one row, TPR
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


def _gp_ranks(keys: np.ndarray, E: int) -> tuple:
    """dispatch_grouped_pull_kernel's stable ranks of one group's entries (ids in
    (token, slot) order, -1 for none), step by step: pass n holds entries
    [1024n, 1024n + 1024), wave w of it lanes [64w, 64w + 64); a lane's rank is its
    id's count in the earlier passes, plus the earlier waves' counts from the byte
    table, plus the lanes before it in its wave holding the same id (the id-bit
    ballots agree on every bit exactly when the ids are equal).  Returns the ranks
    and the group's count per id."""
    NT, WAVES = 1024, 16
    n_ent = len(keys)
    rank = np.full(n_ent, -1, np.int64)
    run = np.zeros(E, np.int64)
    for n in range((n_ent + NT - 1) // NT):
        k = np.full(NT, -1, np.int64)
        part = keys[n * NT:(n + 1) * NT]
        k[:len(part)] = part
        k = k.reshape(WAVES, 64)
        table = np.zeros((E, WAVES), np.int64)  # the byte table: id x wave
        inw = np.zeros((WAVES, 64), np.int64)
        lower = np.tril(np.ones((64, 64), bool), -1)  # lanes before the lane
        for w in range(WAVES):
            kw = k[w]
            eq = (kw[:, None] == kw[None, :]) & (kw[:, None] >= 0)
            inw[w] = (eq & lower).sum(1)
            v = kw[kw >= 0]
            table[:, w] = np.bincount(v, minlength=E)
        assert table.max(initial=0) <= 64  # fits a byte
        before = np.cumsum(table, axis=1) - table  # waves before, per id
        for w in range(WAVES):
            for l in range(64):
                i = n * NT + w * 64 + l
                if i < n_ent and k[w, l] >= 0:
                    rank[i] = run[k[w, l]] + before[k[w, l], w] + inw[w, l]
        run += table.sum(1)
    return rank, run


def _threshold(col: np.ndarray, m: int, Q: int):
    """gp_rank_threshold: the token holding rank r's receive row m (the first one
    dropped), None when the rank keeps all its rows.  off(q) = the rank's tokens in
    the chunks before q = rank_base[q // 4] + rank_off[q]."""
    if m >= col.sum():
        return None
    if m <= 0:
        return 0
    cnt = np.array([col[q * CHUNK:(q + 1) * CHUNK].sum() for q in range(Q)])
    off = np.cumsum(cnt) - cnt
    G4 = (Q + 3) // 4
    rank_base = off[0::4]
    g4 = 0
    for b in range(0, G4, 64):  # batches of 64 groups, lanes over the groups
        le = [b + i < G4 and rank_base[b + i] <= m for i in range(64)]
        if any(le):
            g4 = b + max(i for i in range(64) if le[i])
        if not all(le):
            break
    lq = [i for i in range(4) if 4 * g4 + i < Q and off[4 * g4 + i] <= m]
    qs = 4 * g4 + (max(lq) if lq else 0)
    k = m - off[qs]
    bits = sum(1 << l for l in range(CHUNK) if qs * CHUNK + l < len(col) and col[qs * CHUNK + l])
    assert 0 <= k < bin(bits).count("1")
    return qs * CHUNK + _nth_set_bit(bits, k)


def _check_grouped_pull(idx, E, R, lay, note, dis, row_units, align_sizes, recv_capacity, gcap=None):
    """dispatch_grouped_pull_kernel's positions (segment start + received entries of
    the id before the group + stable rank), its per-XCD base counts, its list and its
    task enumeration, checked against the oracle's grouping of the dispatched rows."""
    T, K = idx.shape
    epr = E // R
    o = oracle.Oracle()
    n_rows = note["num_recv_tokens"]
    grp = o.group_by_expert(np.zeros((n_rows, 8), np.uint16), dis["recv_topk_idx"], dis["recv_topk_weights"],
                            note["recv_gbl_rank_prefix_sum"], align_sizes, E, num_recv_rows=recv_capacity,
                            grouped_capacity=gcap)
    send_slot = dis["send_slot"]
    sizes = np.maximum(align_sizes.astype(np.int64), 0)
    seg = np.cumsum(sizes) - sizes
    total = int(sizes.sum())
    limit = total if gcap is None else min(total, gcap)
    assert grp["num_grouped_rows"] == min(total, 2 ** 31 - 1)
    U = 1 if row_units >= 14 * CHUNK else 2 if row_units >= 7 * CHUNK else 4
    TPR = (row_units + U * CHUNK - 1) // (U * CHUNK)
    W, GT, XCDS_ = 32 * 16, 128, 8
    # received: the token's row on the id's rank exists; per rank that is a prefix of the tokens
    ids = np.where((idx >= 0) & (idx < E), idx, -1)
    rk = np.where(ids >= 0, ids // epr, 0)
    recv = (ids >= 0) & (send_slot[np.arange(T)[:, None], rk] >= 0)
    for r in range(R):
        got = send_slot[:, r] >= 0
        routed = lay["is_token_in_rank"][:, r] != 0
        thr = np.nonzero(routed & ~got)[0]
        if len(thr):
            assert not (got[thr[0]:] & routed[thr[0]:]).any()  # dropped rows are the slab's last
    # the kernel's per-rank token threshold (groups of four chunks, then the chunk,
    # then the token), from the chunk offsets the workspace holds
    slab0 = np.concatenate([[0], note["recv_gbl_rank_prefix_sum"][:-1]]).astype(np.int64)
    Q = (T + CHUNK - 1) // CHUNK
    for r in range(R):
        col = lay["is_token_in_rank"][:, r] != 0
        m = recv_capacity - slab0[r]
        routed = np.nonzero(col)[0]
        want = routed[m] if 0 <= m < len(routed) else (0 if m < 0 else None)
        assert _threshold(col, m, Q) == want, r

    keys_all = np.where(recv, ids, -1).reshape(-1)
    G = (T + GT - 1) // GT

    def count(t0, t1):
        v = keys_all[t0 * K:t1 * K]
        return np.bincount(v[v >= 0], minlength=E)

    issued = {}
    over = False
    base_final = None
    for x in range(XCDS_):
        base = count(0, min(x, G) * GT)  # the prologue: groups before the XCD's first
        for g in range(x, G, XCDS_):
            keys = keys_all[g * GT * K:min((g + 1) * GT, T) * K]
            rank, cnt = _gp_ranks(keys, E)
            pre = np.cumsum(cnt) - cnt
            lst = {}
            for i, e in enumerate(keys):
                if e < 0:
                    continue
                li = base[e] + rank[i]
                pos = seg[e] + li
                placed = li < sizes[e] and pos < limit
                t, j = g * GT + i // K, i % K
                want = grp["slot_pos"][send_slot[t, e // epr], j]
                assert (pos if placed else -1) == want, (t, j, e, pos, want)
                over |= not placed
                lst[pre[e] + rank[i]] = (i // K, pos) if placed else (-1, -1)
            assert sorted(lst) == list(range(int(cnt.sum())))
            tasks = int(cnt.sum()) * TPR
            for wx in range(W):
                for k in _wave_tasks(wx, W, tasks):
                    ent, part = divmod(k, TPR)
                    tl, pos = lst[ent]
                    if tl < 0:
                        continue
                    key = (int(pos), part)
                    assert key not in issued
                    issued[key] = g * GT + tl
            base = base + cnt + count(min((g + 1) * GT, T), min((g + XCDS_) * GT, T))
        if base_final is None:
            base_final = base
        assert np.array_equal(base, base_final)  # every block ends with the same counts
    entries = grp["grouped_row"] >= 0
    assert len(issued) == int(entries.sum()) * TPR
    src = dis["recv_src_info"]
    for pos in np.nonzero(entries)[0][:: max(1, entries.sum() // 2000)]:
        assert issued[(int(pos), 0)] == src[grp["grouped_row"][pos], 1]
    # padding: [start + min(received, size), min(start + size, limit)) of every segment
    pad = np.zeros(len(grp["grouped_row"]), bool)
    for e in range(E):
        lo, hi = seg[e] + min(base_final[e], sizes[e]), min(seg[e] + sizes[e], limit)
        pad[lo:max(lo, hi)] = True
    assert np.array_equal(pad, grp["grouped_row"] == -1)
    return over


@pytest.mark.parametrize("name,align", [("prefill", 4), ("skew", 1), ("large", 8)])
def test_grouped_pull_positions_and_tasks(name, align):
    """dispatch_grouped_pull_kernel on the benchmark's workloads (8 slots: one pass)."""
    d, wl, lay, note, dis = _routing(name)
    aligned = -(-lay["num_tokens_per_expert"] // align) * align
    assert not _check_grouped_pull(d["topk_idx"], wl.experts, wl.ranks, lay, note, dis, wl.hidden * 2 // 16,
                                   aligned, note["num_recv_tokens"])


def test_grouped_pull_many_slots_short_capacities():
    """20 slots a token (three passes of the ranking), duplicates and masked slots,
    receive rows dropped at a short capacity and a short grouped capacity."""
    rng = np.random.default_rng(44)
    T, R, E, K, C = 2300, 16, 128, 20, 5
    idx = np.stack([rng.choice(E, K, replace=True) for _ in range(T)]).astype(np.int64)
    idx.reshape(-1)[rng.choice(T * K, T * K // 10, replace=False)] = -1
    w = rng.random((T, K)).astype(np.float32)
    o = oracle.Oracle()
    lay = o.layout(idx, E, R)
    note = o.notify(lay["is_token_in_rank"], lay["num_tokens_per_rank"], lay["num_tokens_per_rdma_rank"],
                    lay["num_tokens_per_expert"], C, 4)
    cap = note["num_recv_tokens"] - 900
    dis = o.dispatch(np.zeros((T, 8), np.uint16), idx, w, lay["is_token_in_rank"], note["gbl_channel_prefix_matrix"],
                     note["recv_gbl_rank_prefix_sum"], E, recv_capacity=cap)
    aligned = note["num_recv_tokens_per_expert"]
    gcap = int(aligned.sum()) - 500
    assert _check_grouped_pull(idx, E, R, lay, note, dis, 520 * 2 // 16, aligned, cap, gcap=gcap)
