"""Checks that pin the CPU oracle to things other than itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` (the real one, or a variant
built from a planted mistake) and returns a list of failure strings; an empty
list means the pin holds.  The pins are:

* the hand-worked example under ``tests/golden/`` (derived from the definitions
  on the pages, which print no numeric example themselves);
* invariants the definitions imply (counts, totals, monotone prefixes, a row
  bijection, slab and channel segment boundaries, metadata masking);
* closed forms: identity experts return x bit-exactly, power-of-two scaled
  experts return the exact weighted sum within half a bf16 ulp, aligned
  counts equal ceil(n/a)*a;
* brute force over every routing of 1 or 2 tokens on tiny shapes, compared
  with a second formulation written independently here (sets, sorting,
  channel index by integer division);
* the bf16 rounding against torch's own round-to-nearest-even conversion.
"""
from __future__ import annotations

import itertools
import json
import math
import os
from collections import Counter

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "worked_example.json")


def _bf16_from_float(a) -> np.ndarray:
    """Exact floats (small integers, dyadic fractions) to bf16 bit patterns."""
    f = np.asarray(a, dtype=np.float32)
    bits = f.view(np.uint32)
    assert np.all((bits & 0xFFFF) == 0), "value not exact in bf16"
    return (bits >> 16).astype(np.uint16)


def bf16_to_f64(u: np.ndarray) -> np.ndarray:
    return (np.asarray(u, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _eq(name, got, want, errs):
    got = np.asarray(got)
    want = np.asarray(want)
    if got.shape != want.shape or not np.array_equal(got, want):
        errs.append(f"{name}: got {got.tolist()} want {want.tolist()}")


# --------------------------------------------------------------------------- golden
def pin_golden(o) -> list[str]:
    g = json.load(open(GOLDEN))
    s, inp, exp = g["shape"], g["inputs"], g["expected"]
    T, H, K, E, R, C = (s[k] for k in ("tokens", "hidden", "topk", "experts", "ranks", "channels"))
    idx = np.array(inp["topk_idx"], np.int64)
    w = np.array(inp["topk_weights"], np.float32)
    x = _bf16_from_float([[(t + 1) * (i + 1) for i in range(H)] for t in range(T)])
    errs: list[str] = []
    lay = o.layout(idx, E, R)
    for key in ("is_token_in_rank", "num_tokens_per_rank", "num_tokens_per_rdma_rank", "num_tokens_per_expert"):
        _eq(key, lay[key], exp[key], errs)
    note = o.notify(lay["is_token_in_rank"], lay["num_tokens_per_rank"], lay["num_tokens_per_rdma_rank"],
                    lay["num_tokens_per_expert"], C, s["expert_alignment"])
    for key in ("gbl_channel_prefix_matrix", "rdma_channel_prefix_matrix", "recv_gbl_rank_prefix_sum",
                "recv_rdma_rank_prefix_sum", "num_recv_tokens_per_expert", "num_recv_tokens"):
        _eq(key, note[key], exp[key], errs)
    dis = o.dispatch(x, idx, w, lay["is_token_in_rank"], note["gbl_channel_prefix_matrix"],
                     note["recv_gbl_rank_prefix_sum"], E, s["my_rank"])
    for key in ("send_slot", "recv_src_info", "recv_topk_idx", "recv_topk_weights"):
        _eq(key, dis[key], exp[key], errs)
    _eq("recv_x", dis["recv_x"], x[np.array(exp["recv_x_source_token"])], errs)
    n = note["num_recv_tokens"]
    com = o.combine(dis["recv_x"], dis["recv_topk_weights"], dis["send_slot"], n)
    want_id = x.copy()
    want_id[4] = 0
    _eq("combined_x(identity)", com["combined_x"], want_id, errs)
    _eq("combined_topk_weights", com["combined_topk_weights"], exp["combined_topk_weights"], errs)
    y = _bf16_from_float([[s_ + 1] * H for s_ in range(n)])
    com = o.combine(y, dis["recv_topk_weights"], dis["send_slot"], n)
    want = _bf16_from_float([[v] * H for v in exp["combined_x_with_y"]])
    _eq("combined_x(y)", com["combined_x"], want, errs)
    for st, name in ((lay, "layout"), (note, "notify"), (dis, "dispatch"), (com, "combine")):
        if st["status"] != 0:
            errs.append(f"{name} status {st['status']}")
    return errs


# --------------------------------------------------------------------------- invariants
def layout_invariants(idx: np.ndarray, E: int, R: int, lay: dict) -> list[str]:
    errs = []
    T, K = idx.shape
    er = E // R
    nodes = max(1, R // 8)
    in_rank = lay["is_token_in_rank"].astype(np.int64)
    per_rank = lay["num_tokens_per_rank"].astype(np.int64)
    per_node = lay["num_tokens_per_rdma_rank"].astype(np.int64)
    per_exp = lay["num_tokens_per_expert"].astype(np.int64)
    valid = int(((idx >= 0) & (idx < E)).sum())
    if per_exp.sum() != valid:
        errs.append(f"sum(per_expert)={per_exp.sum()} != valid slots {valid}")
    if not np.array_equal(in_rank.sum(0), per_rank):
        errs.append("column sums of is_token_in_rank != num_tokens_per_rank")
    if not set(np.unique(in_rank)).issubset({0, 1}):
        errs.append("is_token_in_rank not boolean")
    by_rank = per_exp.reshape(R, er)
    if np.any(by_rank.max(1) > per_rank) or np.any(per_rank > by_rank.sum(1)):
        errs.append("max_e count <= per_rank <= sum_e count violated")
    for n in range(nodes):
        sl = per_rank[n * 8:(n + 1) * 8]
        if not (sl.max(initial=0) <= per_node[n] <= sl.sum()):
            errs.append(f"node {n}: per-node count {per_node[n]} outside [max, sum] of its ranks")
    # tokens whose every slot is masked reach no rank and no node
    dead = ~((idx >= 0) & (idx < E)).any(1)
    if in_rank[dead].any():
        errs.append("fully masked token routed")
    if np.any(per_node > T - dead.sum()):
        errs.append("a node receives more tokens than there are live tokens")
    return errs


def notify_invariants(lay: dict, note: dict, C: int, align: int) -> list[str]:
    errs = []
    gbl = note["gbl_channel_prefix_matrix"].astype(np.int64)
    rdma = note["rdma_channel_prefix_matrix"].astype(np.int64)
    per_rank = lay["num_tokens_per_rank"]
    per_node = lay["num_tokens_per_rdma_rank"]
    in_rank = lay["is_token_in_rank"]
    T = in_rank.shape[0]
    tc = -(-T // C) if C else 0
    if np.any(np.diff(gbl, axis=1) < 0) or np.any(np.diff(rdma, axis=1) < 0):
        errs.append("channel prefix not monotone")
    if not np.array_equal(gbl[:, -1], per_rank):
        errs.append("gbl last column != per-rank totals")
    if not np.array_equal(rdma[:, -1], per_node):
        errs.append("rdma last column != per-node totals")
    if not np.array_equal(gbl[:, 0], in_rank[:min(tc, T)].astype(np.int64).sum(0)):
        errs.append("gbl first column != channel-0 counts")
    recv = note["recv_gbl_rank_prefix_sum"].astype(np.int64)
    if not np.array_equal(np.diff(np.concatenate([[0], recv])), per_rank):
        errs.append("recv_gbl increments != per-rank counts")
    if note["num_recv_tokens"] != int(per_rank.sum()):
        errs.append("num_recv_tokens != sum per_rank")
    rr = note["recv_rdma_rank_prefix_sum"].astype(np.int64)
    if not np.array_equal(np.diff(np.concatenate([[0], rr])), per_node):
        errs.append("recv_rdma increments != per-node counts")
    n = lay["num_tokens_per_expert"].astype(np.int64)
    a = note["num_recv_tokens_per_expert"].astype(np.int64)
    if np.any(a % align) or np.any(a < n) or np.any(a >= n + align):
        errs.append("aligned per-expert counts not ceil(n/a)*a")
    return errs


def dispatch_invariants(x, idx, w, E, R, C, my_rank, lay, note, dis) -> list[str]:
    errs = []
    T, K = idx.shape
    er = E // R
    n = note["num_recv_tokens"]
    slot = dis["send_slot"].astype(np.int64)
    in_rank = lay["is_token_in_rank"].astype(bool)
    if not np.array_equal(slot >= 0, in_rank):
        errs.append("send_slot >= 0 pattern != is_token_in_rank")
    used = np.sort(slot[slot >= 0])
    if not np.array_equal(used, np.arange(n)):
        errs.append("send_slot is not a bijection onto [0, N)")
        return errs
    tt, rr = np.nonzero(slot >= 0)
    ss = slot[tt, rr]
    src = dis["recv_src_info"]
    if not (np.all(src[ss, 0] == my_rank) and np.array_equal(src[ss, 1], tt)):
        errs.append("src_info does not point back to (my_rank, t)")
    recv = note["recv_gbl_rank_prefix_sum"].astype(np.int64)
    base = np.concatenate([[0], recv[:-1]])
    if np.any(ss < base[rr]) or np.any(ss >= recv[rr]):
        errs.append("row outside its rank's slab")
    # inside a slab, source tokens strictly increase
    order = np.argsort(ss)
    s_rank, s_tok = rr[order], tt[order]
    same = s_rank[1:] == s_rank[:-1]
    if np.any(s_tok[1:][same] <= s_tok[:-1][same]):
        errs.append("source tokens not increasing inside a slab")
    # channel segment boundaries inside each slab
    gbl = note["gbl_channel_prefix_matrix"].astype(np.int64)
    tc = -(-T // C)
    ch = tt // tc if tc else tt
    lo = base[rr] + np.where(ch > 0, gbl[rr, np.maximum(ch - 1, 0)], 0)
    hi = base[rr] + gbl[rr, ch]
    if np.any(ss < lo) or np.any(ss >= hi):
        errs.append("row outside its [rank][channel] segment")
    if x is not None and not np.array_equal(dis["recv_x"][ss], x[tt]):
        errs.append("recv_x row != x[src]")
    # metadata: weights / local ids only for experts living on the receiving rank
    rw = dis["recv_topk_weights"][ss]
    ri = dis["recv_topk_idx"][ss] if dis["recv_topk_idx"] is not None else None
    e = idx[tt]
    on = (e >= 0) & (e < E) & (e // max(er, 1) == rr[:, None])
    if not np.array_equal(rw, np.where(on, w[tt], np.float32(0))):
        errs.append("recv_topk_weights masking wrong")
    if ri is not None:
        if not np.array_equal(ri, np.where(on, e - rr[:, None] * er, -1)):
            errs.append("recv_topk_idx local ids wrong")
        if np.any(ri < -1) or np.any(ri >= er):
            errs.append("recv_topk_idx outside [-1, E/R)")
            return errs
        cnt = np.zeros(E, np.int64)
        valid = ri >= 0
        np.add.at(cnt, (rr[:, None] * er + ri)[valid], 1)
        if not np.array_equal(cnt, lay["num_tokens_per_expert"]):
            errs.append("per-local-expert receive counts != num_tokens_per_expert")
    return errs


def _ulp_bf16(v: np.ndarray) -> np.ndarray:
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, 2.0 ** (e - 7), 2.0 ** -133)


def combine_closed_forms(o, x, idx, w, E, R, lay, note, dis) -> list[str]:
    errs = []
    T, K = idx.shape
    er = E // R
    n = note["num_recv_tokens"]
    # 1) identity experts: combined == x where the token went anywhere, +0 elsewhere
    com = o.combine(dis["recv_x"], dis["recv_topk_weights"], dis["send_slot"], n)
    live = lay["is_token_in_rank"].any(1)
    want = np.where(live[:, None], x, np.uint16(0))
    # weights of a live token sum to 1 only when every valid slot carries weight;
    # the generator's softmax guarantees it.  Compared as values: the
    # accumulator starts at +0, so an x element of -0 comes back as +0.
    got_v, want_v = bf16_to_f64(com["combined_x"]), bf16_to_f64(want)
    if not np.array_equal(got_v, want_v):
        bad = int((got_v != want_v).sum())
        errs.append(f"identity combine != x on {bad} elements")
    valid = (idx >= 0) & (idx < E)
    if not np.array_equal(com["combined_topk_weights"], np.where(valid, w, np.float32(0))):
        errs.append("combined_topk_weights != masked topk_weights")
    # 2) power-of-two scaled experts: y[s] = 2^((r mod 4) - 1) * x[src]
    slot = dis["send_slot"]
    tt, rr = np.nonzero(slot >= 0)
    ss = slot[tt, rr]
    scale = 2.0 ** ((rr % 4) - 1)
    y = np.zeros_like(dis["recv_x"])
    yf = bf16_to_f64(x[tt]) * scale[:, None]
    y[ss] = (yf.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)  # exact: power-of-two scaling
    W = np.zeros((T, R))
    for j in range(K):
        ok = valid[:, j]
        np.add.at(W, (np.nonzero(ok)[0], idx[ok, j] // er), w[ok, j].astype(np.float64))
    coef = (W * (2.0 ** ((np.arange(R) % 4) - 1))[None, :]).sum(1)
    exact = coef[:, None] * bf16_to_f64(x)
    got = bf16_to_f64(o.combine(y, dis["recv_topk_weights"], slot, n)["combined_x"])
    tol = 0.5 * _ulp_bf16(exact) * 1.001
    if np.any(np.abs(got - exact) > tol):
        errs.append(f"scaled combine off by {np.max(np.abs(got - exact) - tol):.3g} beyond half-ulp")
    # 3) the binary64 evaluation of the same sum: the closed form up to the
    # rounding of a few binary64 additions (the products W*y are exact there)
    f64, st = o.combine_f64(y, dis["recv_topk_weights"], slot, n)
    if st != 0 or np.any(np.abs(f64 - exact) > 1e-12 * np.abs(exact) + 1e-300):
        errs.append(f"binary64 combine differs from the closed form by {np.max(np.abs(f64 - exact)):.3g}")
    return errs


# --------------------------------------------------------------------------- brute force
def _second_formulation(idx, E, R, C, my_rank):
    """Independent restatement: destination sets, a sorted (rank, token) list."""
    T, K = idx.shape
    er = E // R
    dest = [sorted({int(e) // er for e in row if 0 <= e < E}) for row in idx]
    nodes = max(1, R // 8)
    tc = -(-T // C) if T else 1
    chan = [t // tc for t in range(T)]
    per_rank = [sum(r in d for d in dest) for r in range(R)]
    per_node = [sum(any(r // 8 == nd for r in d) for d in dest) for nd in range(nodes)]
    cnt = Counter(int(e) for row in idx for e in row if 0 <= e < E)
    per_exp = [cnt[e] for e in range(E)]
    gbl = [[sum(1 for t in range(T) if r in dest[t] and chan[t] <= c) for c in range(C)] for r in range(R)]
    rdma = [[sum(1 for t in range(T) if any(r // 8 == nd for r in dest[t]) and chan[t] <= c)
             for c in range(C)] for nd in range(nodes)]
    pairs = sorted((r, t) for t in range(T) for r in dest[t])
    slot = [[-1] * R for _ in range(T)]
    for i, (r, t) in enumerate(pairs):
        slot[t][r] = i
    return dict(per_rank=per_rank, per_node=per_node, per_exp=per_exp, gbl=gbl, rdma=rdma, slot=slot,
                n=len(pairs), dest=dest)


def pin_bruteforce(o, max_cases: int | None = None) -> list[str]:
    errs: list[str] = []
    rng = np.random.default_rng(7)
    E, K = 4, 2
    slot_vals = [-1, 0, 1, 2, 3]
    rows = [r for r in itertools.product(slot_vals, repeat=K)]
    cases = 0
    for R in (1, 2, 4):
        for T in (1, 2):
            for routing in itertools.product(rows, repeat=T):
                idx = np.array(routing, np.int64).reshape(T, K)
                for C in (1, 2, 3, 5):
                    cases += 1
                    if max_cases and cases > max_cases:
                        return errs
                    ref = _second_formulation(idx, E, R, C, 1)
                    lay = o.layout(idx, E, R)
                    if lay["num_tokens_per_rank"].tolist() != ref["per_rank"] or \
                       lay["num_tokens_per_rdma_rank"].tolist() != ref["per_node"] or \
                       lay["num_tokens_per_expert"].tolist() != ref["per_exp"]:
                        errs.append(f"layout mismatch idx={idx.tolist()} R={R}")
                        continue
                    note = o.notify(lay["is_token_in_rank"], lay["num_tokens_per_rank"],
                                    lay["num_tokens_per_rdma_rank"], lay["num_tokens_per_expert"], C, 1)
                    if note["gbl_channel_prefix_matrix"].tolist() != ref["gbl"] or \
                       note["rdma_channel_prefix_matrix"].tolist() != ref["rdma"]:
                        errs.append(f"notify mismatch idx={idx.tolist()} R={R} C={C}")
                        continue
                    H = 8
                    x = _bf16_from_float(rng.integers(-8, 9, size=(T, H)).astype(np.float32))
                    w = (rng.integers(1, 8, size=(T, K)) / 8.0).astype(np.float32)
                    dis = o.dispatch(x, idx, w, lay["is_token_in_rank"], note["gbl_channel_prefix_matrix"],
                                     note["recv_gbl_rank_prefix_sum"], E, 1)
                    if dis["send_slot"].tolist() != ref["slot"]:
                        errs.append(f"dispatch slots mismatch idx={idx.tolist()} R={R} C={C}")
                        continue
                    n = ref["n"]
                    y = _bf16_from_float(rng.integers(-8, 9, size=(max(n, 1), H)).astype(np.float32))[:n]
                    com = o.combine(y, dis["recv_topk_weights"], dis["send_slot"], n)
                    er = E // R
                    want = np.zeros((T, H))
                    for t in range(T):
                        for r in ref["dest"][t]:
                            wsum = sum(float(w[t, j]) for j in range(K) if 0 <= idx[t, j] < E and idx[t, j] // er == r)
                            want[t] += wsum * bf16_to_f64(y[ref["slot"][t][r]])
                    got = bf16_to_f64(com["combined_x"])
                    if np.any(np.abs(got - want) > 0.5 * _ulp_bf16(want) * 1.001):
                        errs.append(f"combine mismatch idx={idx.tolist()} R={R} C={C}")
                    # the binary64 form: small integers times multiples of 1/8, so
                    # every partial sum is exact and the results must be equal
                    f64, st = o.combine_f64(y, dis["recv_topk_weights"], dis["send_slot"], n)
                    if st != 0 or not np.array_equal(f64, want):
                        errs.append(f"binary64 combine mismatch idx={idx.tolist()} R={R} C={C}")
    return errs


# --------------------------------------------------------------------------- bf16 rounding
def pin_bf16_rounding(o) -> list[str]:
    import torch

    rng = np.random.default_rng(3)
    vals = [rng.standard_normal(20000).astype(np.float32),
            (rng.standard_normal(20000) * 1e30).astype(np.float32),
            (rng.standard_normal(2000) * 1e-40).astype(np.float32)]
    # exact ties: kept bits odd/even with dropped half exactly 0x8000
    base = rng.integers(0, 1 << 15, size=4000, dtype=np.uint32) << 16
    base = base[(base & 0x7F800000) != 0x7F800000]  # NaN payloads are implementation-defined
    ties = (base | 0x8000).view(np.float32)
    specials = np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38, -3.3895314e38, 1.0, -1.0], np.float32)
    f = np.concatenate(vals + [ties, specials])
    got = o.bf16_round(f)
    want = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    errs = []
    if not np.array_equal(got, want):
        errs.append(f"bf16 rounding differs from torch on {int((got != want).sum())} values")
    nan = o.bf16_round(np.array([np.nan], np.float32))
    if not ((nan[0] & 0x7F80) == 0x7F80 and (nan[0] & 0x7F) != 0):
        errs.append("NaN not kept as NaN")
    return errs


# --------------------------------------------------------------------------- whole-workload pin
def pin_workload(o, inputs: dict, hidden: int | None = None) -> list[str]:
    """All invariants and closed forms on one generated workload.  ``hidden``
    narrows x (slot logic does not depend on it) to keep CPU runs short."""
    wl = inputs["workload"]
    x = inputs["x"]
    if hidden is not None and x is not None:
        x = np.ascontiguousarray(x[:, :hidden])
    idx, w = inputs["topk_idx"], inputs["topk_weights"]
    E, R, C = wl.experts, wl.ranks, wl.channels
    errs = []
    lay = o.layout(idx, E, R)
    errs += layout_invariants(idx, E, R, lay)
    note = o.notify(lay["is_token_in_rank"], lay["num_tokens_per_rank"], lay["num_tokens_per_rdma_rank"],
                    lay["num_tokens_per_expert"], C, wl.expert_alignment)
    errs += notify_invariants(lay, note, C, wl.expert_alignment)
    if x is None:
        return errs
    dis = o.dispatch(x, idx, w, lay["is_token_in_rank"], note["gbl_channel_prefix_matrix"],
                     note["recv_gbl_rank_prefix_sum"], E, 0)
    errs += dispatch_invariants(x, idx, w, E, R, C, 0, lay, note, dis)
    if not errs:
        errs += combine_closed_forms(o, x, idx, w, E, R, lay, note, dis)
    for st, name in ((lay, "layout"), (note, "notify"), (dis, "dispatch")):
        if st["status"] != 0:
            errs.append(f"{name} status {st['status']}")
    return errs


def pin_dispatch_prefix_checks(o, inputs: dict) -> list[str]:
    """Dispatch flags prefixes that disagree with is_token_in_rank: entries of the
    channel prefix matrix (first, middle and last columns) and receive prefixes are
    moved by one in turn, and each must raise the count-mismatch bit.  A moved
    channel prefix must leave the rows as they were (they follow the walk; a receive
    prefix is where a slab starts, so it does move rows)."""
    import oracle as _oracle

    wl = inputs["workload"]
    x = np.ascontiguousarray(inputs["x"][:, :16])
    idx, w = inputs["topk_idx"], inputs["topk_weights"]
    E, R, C = wl.experts, wl.ranks, wl.channels
    lay = o.layout(idx, E, R)
    note = o.notify(lay["is_token_in_rank"], lay["num_tokens_per_rank"], lay["num_tokens_per_rdma_rank"],
                    lay["num_tokens_per_expert"], C, 1)
    gbl, recv = note["gbl_channel_prefix_matrix"], note["recv_gbl_rank_prefix_sum"]
    base = o.dispatch(x, idx, w, lay["is_token_in_rank"], gbl, recv, E)
    errs = [] if base["status"] == 0 else [f"consistent prefixes flagged: {base['status']}"]
    edits = [("gbl", r, c) for r in (0, R - 1) for c in (0, C // 2, C - 1)] + [("recv", r, 0) for r in (0, R - 1)]
    for kind, r, c in edits:
        g2, rv2 = gbl.copy(), recv.copy()
        if kind == "gbl":
            g2[r, c] += 1
        else:
            rv2[r] += 1
        d = o.dispatch(x, idx, w, lay["is_token_in_rank"], g2, rv2, E, recv_capacity=int(recv[-1]) + 1)
        if not d["status"] & _oracle.COUNT_MISMATCH:
            errs.append(f"{kind}[{r}][{c}] + 1 not flagged")
        n = int(recv[-1])
        if kind == "gbl" and not np.array_equal(d["send_slot"], base["send_slot"]) or \
                kind == "gbl" and not np.array_equal(d["recv_x"][:n], base["recv_x"]):
            errs.append(f"{kind}[{r}][{c}] + 1 moved the rows")
    return errs


def pin_count_checks_and_overflow(o, inputs: dict) -> list[str]:
    """Notify's counts must be the map's: with consistent inputs its status is 0, and a per-rank or per-node
    count moved by one (first and last rank, first and last node) must raise the count-mismatch bit.  A
    receive capacity below N drops exactly the rows the full dispatch put at or past it: the status is the
    overflow bit alone (the prefixes still agree with the map), the kept rows and their metadata are the
    full dispatch's, and send_slot keeps exactly the entries below the capacity."""
    import oracle as _oracle

    wl = inputs["workload"]
    x = np.ascontiguousarray(inputs["x"][:, :16])
    idx, w = inputs["topk_idx"], inputs["topk_weights"]
    E, R, C = wl.experts, wl.ranks, wl.channels
    nodes = max(1, R // 8)
    lay = o.layout(idx, E, R)
    args = (lay["is_token_in_rank"], lay["num_tokens_per_rank"], lay["num_tokens_per_rdma_rank"],
            lay["num_tokens_per_expert"], C, 1)
    note = o.notify(*args)
    errs = [] if note["status"] == 0 else [f"consistent counts flagged: {note['status']}"]
    for which, i in [("rank", 0), ("rank", R - 1), ("node", 0), ("node", nodes - 1)]:
        per_rank, per_node = lay["num_tokens_per_rank"].copy(), lay["num_tokens_per_rdma_rank"].copy()
        (per_rank if which == "rank" else per_node)[i] += 1
        st = o.notify(lay["is_token_in_rank"], per_rank, per_node, lay["num_tokens_per_expert"], C, 1)["status"]
        if not st & _oracle.COUNT_MISMATCH:
            errs.append(f"notify: {which} count {i} + 1 not flagged")
    gbl, recv = note["gbl_channel_prefix_matrix"], note["recv_gbl_rank_prefix_sum"]
    full = o.dispatch(x, idx, w, lay["is_token_in_rank"], gbl, recv, E)
    n = int(recv[-1])
    cap = n - 10
    d = o.dispatch(x, idx, w, lay["is_token_in_rank"], gbl, recv, E, recv_capacity=cap)
    if d["status"] != _oracle.RECV_OVERFLOW:
        errs.append(f"overflow status {d['status']}, want the overflow bit alone")
    want_slot = np.where(full["send_slot"] < cap, full["send_slot"], -1)
    if not np.array_equal(d["send_slot"], want_slot):
        errs.append("overflow: send_slot differs from the full dispatch's entries below the capacity")
    for k in ("recv_x", "recv_topk_weights", "recv_topk_idx", "recv_src_info"):
        if not np.array_equal(d[k][:cap], full[k][:cap]):
            errs.append(f"overflow: {k} of the kept rows differs")
    return errs


def pin_fp8_and_cached(o, inputs: dict, hidden: int | None = None) -> list[str]:
    """fp8 dispatch moves the fp8 rows and their scales to the rows the bf16
    routing defines; cached dispatch reproduces a full dispatch from its
    send_slot, and a random injective send_slot places row t at exactly the
    rows it names (numpy assignment as the independent formulation)."""
    from combine_ep_get_02_amd.inputs import fp8_rows

    wl = inputs["workload"]
    x = inputs["x"] if hidden is None else np.ascontiguousarray(inputs["x"][:, :hidden])
    idx, w = inputs["topk_idx"], inputs["topk_weights"]
    E, R, C = wl.experts, wl.ranks, wl.channels
    errs = []
    x8, sc = fp8_rows(x)
    lay = o.layout(idx, E, R)
    note = o.notify(lay["is_token_in_rank"], lay["num_tokens_per_rank"], lay["num_tokens_per_rdma_rank"],
                    lay["num_tokens_per_expert"], C, 1)
    args = (idx, w, lay["is_token_in_rank"], note["gbl_channel_prefix_matrix"], note["recv_gbl_rank_prefix_sum"], E)
    d16 = o.dispatch(x, *args)
    d8 = o.dispatch_fp8(x8, sc, *args)
    for k in ("send_slot", "recv_topk_weights", "recv_topk_idx", "recv_src_info"):
        if not np.array_equal(d16[k], d8[k]):
            errs.append(f"fp8 dispatch {k} differs from the bf16 routing")
    slot = d8["send_slot"]
    tt, rr = np.nonzero(slot >= 0)
    ss = slot[tt, rr]
    if not np.array_equal(d8["recv_x"][ss], x8[tt]):
        errs.append("fp8 recv_x row != x8[src]")
    if not np.array_equal(d8["recv_x_scales"][ss], sc[tt]):
        errs.append("fp8 recv_x_scales != x_scales[src]")
    n = note["num_recv_tokens"]
    c16 = o.dispatch_cached(x, slot, n)
    if not np.array_equal(c16["recv_x"], d16["recv_x"]) or c16["status"]:
        errs.append("cached bf16 dispatch != full dispatch")
    c8 = o.dispatch_cached(x8, slot, n, sc)
    if not np.array_equal(c8["recv_x"], d8["recv_x"]) or not np.array_equal(c8["recv_x_scales"], d8["recv_x_scales"]):
        errs.append("cached fp8 dispatch != full dispatch")
    # random injective map with some bad entries
    rng = np.random.default_rng(5)
    T = x.shape[0]
    cap = T * 2
    rs = np.full((T, R), -1, np.int32)
    picks = rng.choice(T * R, min(cap, T * R), replace=False)
    rs.reshape(-1)[picks] = rng.permutation(cap)[: len(picks)]
    rs[0, 0] = cap + 3
    rs[min(1, T - 1), R - 1] = -5
    want = np.zeros((cap,) + x.shape[1:], x.dtype)
    ok = rs >= 0
    ok &= rs < cap
    tt, rr = np.nonzero(ok)
    want[rs[tt, rr]] = x[tt]
    got = o.dispatch_cached(x, rs, cap)
    if not np.array_equal(got["recv_x"], want) or got["status"] != 8:
        errs.append("cached dispatch with a random map is wrong")
    return errs


def pin_golden_grouping(o) -> list[str]:
    """The grouping of the hand-worked example, at alignment 2 and 1 (values
    derived by hand in golden/worked_example.md)."""
    g = json.load(open(GOLDEN))
    s, exp = g["shape"], g["expected"]
    K, E = s["topk"], s["experts"]
    idx = np.array(exp["recv_topk_idx"], np.int64)
    w = np.array(exp["recv_topk_weights"], np.float32)
    n = exp["num_recv_tokens"]
    rows = np.arange(n * 8, dtype=np.int16).reshape(n, 8)  # row s holds 8s .. 8s+7
    errs: list[str] = []
    for align, key in ((2, "alignment_2"), (1, "alignment_1")):
        want = exp["grouping"][key]
        aligned = [(c + align - 1) // align * align for c in exp["num_tokens_per_expert"]]
        got = o.group_by_expert(rows, idx, w, exp["recv_gbl_rank_prefix_sum"], aligned, E)
        _eq(f"{key}: num_grouped_rows", got["num_grouped_rows"], want["num_grouped_rows"], errs)
        _eq(f"{key}: grouped_row", got["grouped_row"], want["grouped_row"], errs)
        _eq(f"{key}: grouped_weights", got["grouped_weights"], want["grouped_weights"], errs)
        _eq(f"{key}: slot_pos", got["slot_pos"], want["slot_pos"], errs)
        gr = np.array(want["grouped_row"])
        want_x = np.where(gr[:, None] >= 0, rows[np.maximum(gr, 0)], 0)
        _eq(f"{key}: grouped_x", got["grouped_x"], want_x, errs)
        if got["status"] != 0:
            errs.append(f"{key}: status {got['status']}")
    return errs


def _grouping_by_sorting(idx, gbl, aligned, er, num_rows, cap):
    """Second formulation of the grouping: list every (expert, row, slot) with
    a valid local id, sort the triples with Python's sort, and lay the segments
    out at the running sums of the aligned sizes."""
    triples = []
    lo = 0
    for r, hi in enumerate(gbl):
        for row in range(lo, min(int(hi), num_rows)):
            for j, le in enumerate(idx[row]):
                if 0 <= le < er:
                    triples.append((r * er + int(le), row, j))
        lo = min(int(hi), num_rows)
    triples.sort()
    start = np.concatenate([[0], np.cumsum(aligned)])
    grow = np.full(cap, -2, np.int64)
    pos = np.full(idx.shape, -1, np.int64)
    seen = Counter()
    overflow = False
    for e, row, j in triples:
        i = seen[e]
        seen[e] += 1
        p = start[e] + i
        if i >= aligned[e] or p >= cap:
            overflow = True
            continue
        grow[p] = row
        pos[row, j] = p
    for e in range(len(aligned)):
        for i in range(seen[e], aligned[e]):
            if start[e] + i < cap:
                grow[start[e] + i] = -1
    return grow, pos, int(start[-1]), overflow


def pin_group_by_expert(o, inputs: dict, align: int, hidden: int | None = None) -> list[str]:
    """Grouping on a workload's real routing: equal to the sorting formulation;
    each segment's entries are exactly the source tokens that chose that
    expert (read back through src_info and the source topk ids), rows
    ascending; sizes equal the layout's per-expert counts; padding is zero;
    then a short grouped capacity and a too-small segment size are flagged."""
    wl = inputs["workload"]
    x = inputs["x"] if hidden is None else np.ascontiguousarray(inputs["x"][:, :hidden])
    idx, w = inputs["topk_idx"], inputs["topk_weights"]
    E, R, C = wl.experts, wl.ranks, wl.channels
    er = E // R
    errs: list[str] = []
    lay = o.layout(idx, E, R)
    note = o.notify(lay["is_token_in_rank"], lay["num_tokens_per_rank"], lay["num_tokens_per_rdma_rank"],
                    lay["num_tokens_per_expert"], C, align)
    dis = o.dispatch(x, idx, w, lay["is_token_in_rank"], note["gbl_channel_prefix_matrix"],
                     note["recv_gbl_rank_prefix_sum"], E)
    n = note["num_recv_tokens"]
    aligned = note["num_recv_tokens_per_expert"].astype(np.int64)
    ridx, rw = dis["recv_topk_idx"][:n], dis["recv_topk_weights"][:n]
    got = o.group_by_expert(dis["recv_x"][:n], ridx, rw, note["recv_gbl_rank_prefix_sum"], aligned, E)
    m = int(aligned.sum())
    grow, pos, m2, _ = _grouping_by_sorting(ridx, note["recv_gbl_rank_prefix_sum"], aligned, er, n, m)
    if got["num_grouped_rows"] != m or m2 != m:
        errs.append("num_grouped_rows != sum of the aligned counts")
    if not np.array_equal(got["grouped_row"], grow) or not np.array_equal(got["slot_pos"], pos):
        errs.append("grouping differs from the sorting formulation")
    live = grow >= 0
    if not np.array_equal(got["grouped_x"][live], dis["recv_x"][grow[live]]) or np.any(got["grouped_x"][~live] != 0):
        errs.append("grouped_x rows wrong or padding not zero")
    rr, jj = np.nonzero(pos >= 0)
    if not np.array_equal(got["grouped_weights"][pos[rr, jj]], rw[rr, jj]) or np.any(got["grouped_weights"][~live] != 0):
        errs.append("grouped weights wrong")
    # source side: segment e holds, rows ascending, one entry per source slot (t, j) with topk_idx == e
    start = np.concatenate([[0], np.cumsum(aligned)])
    src_t = dis["recv_src_info"][:, 1]
    for e in range(E):
        seg = got["grouped_row"][start[e]:start[e + 1]]
        ent = seg[seg >= 0]
        if len(ent) != lay["num_tokens_per_expert"][e]:
            errs.append(f"expert {e}: {len(ent)} entries, layout counted {lay['num_tokens_per_expert'][e]}")
            break
        if np.any(np.diff(ent) < 0):
            errs.append(f"expert {e}: rows not ascending")
            break
        want_t = Counter(int(t) for t in np.nonzero(idx == e)[0])
        if Counter(int(src_t[r]) for r in ent) != want_t:
            errs.append(f"expert {e}: source tokens differ from the tokens that chose it")
            break
        if len(ent) and not np.all((ent >= (note["recv_gbl_rank_prefix_sum"][e // er - 1] if e // er else 0))
                                   & (ent < note["recv_gbl_rank_prefix_sum"][e // er])):
            errs.append(f"expert {e}: an entry outside slab {e // er}")
            break
    if got["status"] != 0:
        errs.append(f"status {got['status']}")
    # rows past the last slab are capacity slack: their ids (here out of range) are not read
    slack_idx = np.concatenate([ridx, np.full((3, ridx.shape[1]), er + 5, np.int64)])
    slack_x = np.concatenate([dis["recv_x"][:n], dis["recv_x"][:3]])
    slack_w = np.concatenate([rw, np.ones((3, rw.shape[1]), np.float32)])
    slack = o.group_by_expert(slack_x, slack_idx, slack_w, note["recv_gbl_rank_prefix_sum"], aligned, E)
    if slack["status"] != 0 or not np.array_equal(slack["grouped_row"], got["grouped_row"]) or \
            np.any(slack["slot_pos"][n:] != -1):
        errs.append("capacity slack rows were read")
    # a short grouped capacity and one segment sized too small: flagged, the rest as the formulation says
    small = aligned.copy()
    e_big = int(np.argmax(lay["num_tokens_per_expert"]))
    small[e_big] = max(0, small[e_big] - align - 1)
    cap = max(0, int(small.sum()) - 3)
    got = o.group_by_expert(dis["recv_x"][:n], ridx, rw, note["recv_gbl_rank_prefix_sum"], small, E,
                            grouped_capacity=cap)
    grow, pos, _, over = _grouping_by_sorting(ridx, note["recv_gbl_rank_prefix_sum"], small, er, n, cap)
    if not over or got["status"] != 2:
        errs.append(f"overflow not flagged (status {got['status']})")
    if not np.array_equal(got["grouped_row"], grow) or not np.array_equal(got["slot_pos"], pos):
        errs.append("grouping with overflow differs from the sorting formulation")
    return errs


def expected_ranks_per_token(E: int, R: int, K: int) -> float:
    """Closed form for uniform routing without replacement: R*(1 - C(E-E/R, K)/C(E, K))."""
    er = E // R
    return R * (1.0 - math.comb(E - er, K) / math.comb(E, K))


# --------------------------------------------------------------------------- fp8 (E4M3) quantiser
def _torch_e4m3_values() -> np.ndarray:
    """The value of every E4M3 pattern by torch's own float8_e4m3fn decoding (NaN where torch says so)."""
    import torch

    return torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _torch_e4m3_codes(v: np.ndarray) -> np.ndarray:
    """torch's float8_e4m3fn cast (nearest, ties to even) as bit patterns; exact inside [-448, 448]."""
    import torch

    return torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _e4m3_probe_values(rng) -> np.ndarray:
    """Binary32 values inside [-448, 448]: every finite bf16 pattern there, every midpoint between
    neighbouring E4M3 values and one binary32 step either side of it, and log-uniform randoms."""
    allbf = (np.arange(1 << 16, dtype=np.uint32) << 16).view(np.float32)
    allbf = allbf[np.isfinite(allbf) & (np.abs(allbf) <= 448)]
    pos = np.sort(_torch_e4m3_values()[:0x7F])  # 0 .. 448, the non-negative finite values
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)  # exact in binary32
    near = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(448))])
    rnd = (np.exp2(rng.uniform(-14, 8.8, 200000)) * rng.choice([-1.0, 1.0], 200000)).astype(np.float32)
    rnd = rnd[np.abs(rnd) <= 448]
    return np.concatenate([allbf, near, -near, rnd, np.array([0.0, -0.0, 448, -448], np.float32)])


def pin_e4m3(o) -> list[str]:
    """The oracle's E4M3 decode against torch's for all 256 patterns; its encode against torch's
    cast over every bf16 value, every tie and random values in range; and against a brute-force
    nearest-value search (ties to the even pattern) that shares nothing with either."""
    errs = []
    want_vals = _torch_e4m3_values()
    got_vals = o.e4m3_decode(np.arange(256, dtype=np.uint8))
    same = (got_vals == want_vals) | (np.isnan(got_vals) & np.isnan(want_vals))
    if not same.all():
        errs.append(f"E4M3 decode differs from torch at patterns {np.flatnonzero(~same)[:8].tolist()}")
    rng = np.random.default_rng(11)
    v = _e4m3_probe_values(rng)
    got = o.e4m3_encode(v)
    want = _torch_e4m3_codes(v)
    if not np.array_equal(got, want):
        bad = np.flatnonzero(got != want)
        errs.append(f"E4M3 encode differs from torch on {bad.size} values, e.g. {v[bad[:4]].tolist()}")
    # brute force on a sample: the nearest finite value, the even pattern on a tie, the sign kept
    s = np.concatenate([v[rng.choice(v.size, 6000, replace=False)], v[-4:]])
    table = want_vals.copy()
    finite = np.flatnonzero(~np.isnan(table))
    dist = np.abs(table[finite][None, :] - s.astype(np.float64)[:, None])
    best = dist.min(axis=1)
    c = o.e4m3_encode(s)
    cval = o.e4m3_decode(c)
    if not np.array_equal(np.abs(cval - s.astype(np.float64)), best):
        errs.append("E4M3 encode is not the nearest value")
    tie = (dist == best[:, None]).sum(axis=1) > 1
    nz = cval != 0  # both signed zeros tie at 0: the sign rule below decides those
    if np.any((c[tie & nz] & 1) != 0):
        errs.append("E4M3 tie not broken to the even pattern")
    if not np.array_equal(c >> 7, np.signbit(s).astype(np.uint8)):
        errs.append("E4M3 sign bit is not the sign of the input")
    return errs


def quantize_groups(rng, rows: int, hidden: int, num_scales: int) -> np.ndarray:
    """bf16 rows whose groups of hidden/num_scales channels span the binary32 exponent range: each group
    is normal values at its own power-of-two scale 2^[-120, 120], and a few groups are special (all zero,
    signed zeros, one non-zero value, bf16 subnormals, a huge spread, a largest value exactly 448)."""
    g = hidden // num_scales
    e = rng.integers(-120, 121, size=(rows, num_scales, 1)).astype(np.float64)
    x = (rng.standard_normal((rows, num_scales, g)) * np.exp2(e)).astype(np.float32)
    x = x.reshape(rows * num_scales, g)
    n = x.shape[0]
    picks = rng.choice(n, size=min(n, 7), replace=False)
    specials = [np.zeros(g, np.float32),
                np.where(np.arange(g) % 2 == 0, 0.0, -0.0).astype(np.float32),
                np.where(np.arange(g) == g // 2, -3.5, 0.0).astype(np.float32),
                (rng.standard_normal(g) * 1e-39).astype(np.float32),
                (rng.standard_normal(g) * np.exp2(rng.integers(-60, 60, g))).astype(np.float32),
                np.concatenate([[448.0], rng.uniform(-448, 448, g - 1)]).astype(np.float32),
                np.concatenate([rng.uniform(-300, 300, g - 1), [-448.0]]).astype(np.float32)]
    for p, sp in zip(picks, specials):
        x[p] = sp
    bits = x.view(np.uint32)
    return (bits >> 16).astype(np.uint16).reshape(rows, hidden)  # truncation gives exact bf16 values


def pin_quantize(o) -> list[str]:
    """Properties the quantiser's reading fixes, none of them its formula retyped: the largest
    magnitude of a group lands on +-448; the round trip value(code) * scale stays within half an E4M3
    step of x (relative 2^-4, or 2^-10 scales in the subnormal range); scaling a group by a power of two
    scales its scale alike and keeps its codes; a group whose largest value is 448 has scale 1 and
    torch's own codes; an all-zero group has zero codes and a positive finite scale; and the
    dequantiser matches torch's float8 -> bf16 conversion at scale 1 and a power-of-two scale."""
    import torch

    errs = []
    rng = np.random.default_rng(12)
    for rows, hidden, S in ((37, 256, 2), (5, 2048, 16), (3, 64, 4), (2, 1024, 1)):
        g = hidden // S
        x = quantize_groups(rng, rows, hidden, S)
        codes, scales = o.quantize_e4m3(x, S)
        xf = bf16_to_f64(x).reshape(rows, S, g)
        cv = o.e4m3_decode(codes).reshape(rows, S, g)
        sc = scales.astype(np.float64)[:, :, None]
        amax = np.abs(xf).max(axis=2)
        live = amax >= 2.0 ** -64
        top = np.abs(xf) == amax[:, :, None]
        if not np.all(np.abs(cv[top & live[:, :, None]]) == 448):
            errs.append(f"quantize {rows}x{hidden}/{S}: a group's largest value is not coded +-448")
        if not np.all((cv[amax == 0] == 0)) or not np.all(np.isfinite(scales)) or not np.all(scales > 0):
            errs.append(f"quantize {rows}x{hidden}/{S}: an all-zero group is not zero codes with a positive scale")
        err = np.abs(cv * sc - xf)
        bound = (2.0 ** -4 + 2.0 ** -20) * np.abs(xf) + 2.0 ** -10 * sc * (1 + 2.0 ** -20)
        if not np.all(err <= bound):
            errs.append(f"quantize {rows}x{hidden}/{S}: round-trip error above half an E4M3 step")
        if not np.array_equal(np.signbit(cv), np.signbit(xf)):
            errs.append(f"quantize {rows}x{hidden}/{S}: code sign differs from x")
        # power-of-two invariance, on groups well above the 2^-64 floor with no bf16 subnormal
        # (so that the scaling is exact)
        k = 5
        e = rng.integers(-50, 91, size=(rows, S, 1)).astype(np.float64)
        xm = (rng.standard_normal((rows, S, g)) * np.exp2(e)).astype(np.float32).reshape(rows, hidden)
        xm_bits = (xm.view(np.uint32) >> 16).astype(np.uint16)
        xs = (bf16_to_f64(xm_bits) * 2.0 ** k).astype(np.float32)
        xs_bits = (xs.view(np.uint32) >> 16).astype(np.uint16)
        c1, s1 = o.quantize_e4m3(xm_bits, S)
        c2, s2 = o.quantize_e4m3(xs_bits, S)
        if not (np.array_equal(c2, c1) and np.array_equal(s2, s1 * np.float32(2.0 ** k))):
            errs.append(f"quantize {rows}x{hidden}/{S}: not invariant under a power-of-two scaling")
    # largest value exactly 448: scale 1, codes as torch's cast of x itself
    g = 128
    x448 = np.concatenate([[448.0], rng.uniform(-448, 448, g - 1)]).astype(np.float32)
    xb = (x448.view(np.uint32) >> 16).astype(np.uint16)[None, :]
    c448, s448 = o.quantize_e4m3(xb, 1)
    if s448[0, 0] != 1.0 or not np.array_equal(c448[0], _torch_e4m3_codes(bf16_to_f64(xb[0]).astype(np.float32))):
        errs.append("quantize: a group whose largest value is 448 is not torch's cast with scale 1")
    # dequantiser: every finite pattern at scale 1 and 2^-7, against torch's conversions
    pats = np.arange(256, dtype=np.uint8)
    pats = pats[(pats & 0x7F) != 0x7F]
    for sc in (1.0, 2.0 ** -7):
        got = o.dequantize_e4m3(pats[None, :], np.array([[sc]], np.float32))[0]
        want = (torch.from_numpy(pats.copy()).view(torch.float8_e4m3fn).to(torch.float32) * sc).to(torch.bfloat16)
        if not np.array_equal(got, want.view(torch.int16).numpy().view(np.uint16)):
            errs.append(f"dequantize at scale {sc} differs from torch's conversion")
    # round trip through the dequantiser: within half an E4M3 step plus half a bf16 step
    x = quantize_groups(rng, 9, 512, 4)
    codes, scales = o.quantize_e4m3(x, 4)
    back = bf16_to_f64(o.dequantize_e4m3(codes, scales))
    xf = bf16_to_f64(x)
    sc = np.repeat(scales.astype(np.float64), 128, axis=1)
    bound = (2.0 ** -4 + 2.0 ** -8 + 2.0 ** -11) * np.abs(xf) + 2.0 ** -9 * sc
    if not np.all(np.abs(back - xf) <= bound):
        errs.append("dequantize(quantize(x)) strays from x")
    return errs


# --------------------------------------------------------------------------- status bits
def pin_flags(o) -> list[str]:
    """Each status bit fires where the definitions put it, and the offending item is skipped exactly as if it
    were masked: topk ids outside [-1, E) in layout; send_slot entries outside [-1, N) in combine (N itself
    included); a local id outside [-1, E/R) in a slab row of the grouping.  Consistent inputs raise nothing.
    Combined weights start from zero whatever the output buffer held before."""
    import ctypes

    import oracle as _oracle

    errs = []
    rng = np.random.default_rng(21)
    T, K, E, R, C, H = 40, 4, 16, 4, 3, 16
    idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int64)
    bad = idx.copy()
    bad[3, 1], bad[7, 0], bad[9, 3] = E, -2, E + 5
    masked = bad.copy()
    masked[3, 1] = masked[7, 0] = masked[9, 3] = -1
    lb, lm = o.layout(bad, E, R), o.layout(masked, E, R)
    if lb["status"] != _oracle.BAD_TOPK_IDX or lm["status"] != 0:
        errs.append(f"layout status {lb['status']} / {lm['status']}, want the bad-id bit / 0")
    for k in ("num_tokens_per_rank", "num_tokens_per_rdma_rank", "num_tokens_per_expert", "is_token_in_rank"):
        if not np.array_equal(lb[k], lm[k]):
            errs.append(f"layout: a bad id not treated as masked in {k}")
    # combine: entries at N, below -1 and past N skipped and flagged
    note = o.notify(lm["is_token_in_rank"], lm["num_tokens_per_rank"], lm["num_tokens_per_rdma_rank"],
                    lm["num_tokens_per_expert"], C, 1)
    x = _bf16_from_float(rng.integers(-8, 8, size=(T, H)).astype(np.float32))
    w = rng.random((T, K)).astype(np.float32)
    d = o.dispatch(x, masked, w, lm["is_token_in_rank"], note["gbl_channel_prefix_matrix"],
                   note["recv_gbl_rank_prefix_sum"], E)
    n = note["num_recv_tokens"]
    y = _bf16_from_float(rng.integers(-8, 8, size=(n, H)).astype(np.float32))
    ss = d["send_slot"].copy()
    free = np.argwhere(ss == -1)
    used = np.argwhere(ss >= 0)
    ss_bad = ss.copy()
    ss_bad[tuple(free[0])] = n
    ss_bad[tuple(free[1])] = -2
    ss_bad[tuple(used[0])] = n + 3
    ss_ref = np.where((ss_bad < -1) | (ss_bad >= n), -1, ss_bad).astype(np.int32)
    # one more row of data past N in y and the weights: an entry equal to N must not reach it
    y_ext = np.vstack([y, _bf16_from_float(np.full((1, H), 3.0, np.float32))])
    w_ext = np.vstack([d["recv_topk_weights"], np.full((1, K), 0.5, np.float32)])
    cb, cr = o.combine(y_ext, w_ext, ss_bad, n), o.combine(y_ext, w_ext, ss_ref, n)
    if cb["status"] != _oracle.BAD_SEND_SLOT or cr["status"] != 0:
        errs.append(f"combine status {cb['status']} / {cr['status']}, want the bad-slot bit / 0")
    ss_n = ss.copy()
    ss_n[tuple(free[0])] = n
    if o.combine(y_ext, w_ext, ss_n, n)["status"] != _oracle.BAD_SEND_SLOT:
        errs.append("combine: an entry equal to N not flagged")
    if not (np.array_equal(cb["combined_x"], cr["combined_x"]) and
            np.array_equal(cb["combined_topk_weights"], cr["combined_topk_weights"])):
        errs.append("combine: a bad slot not skipped")
    # combined weights start from zero: the same call with output buffers full of stale values
    recv_w = np.ascontiguousarray(d["recv_topk_weights"], dtype=np.float32)
    out = np.full((T, H), 0x3F80, np.uint16)
    cw = np.full((T, K), 7.0, np.float32)
    scratch = np.full(H, 5.0, np.float32)
    p = lambda a: a.ctypes.data_as(ctypes.c_void_p)  # noqa: E731
    o.lib.oracle_combine(T, H, K, R, n, p(np.ascontiguousarray(y)), p(recv_w), p(ss_ref), p(out), p(cw), p(scratch))
    if not (np.array_equal(out, cr["combined_x"]) and np.array_equal(cw, cr["combined_topk_weights"])):
        errs.append("combine: outputs depend on what the output buffers held")
    # grouping: a bad local id in a slab row is flagged and skipped like a masked slot
    note4 = o.notify(lm["is_token_in_rank"], lm["num_tokens_per_rank"], lm["num_tokens_per_rdma_rank"],
                     lm["num_tokens_per_expert"], C, 4)
    ridx = d["recv_topk_idx"].copy()
    row, j = np.argwhere(ridx >= 0)[5]
    ridx_bad, ridx_masked = ridx.copy(), ridx.copy()
    ridx_bad[row, j], ridx_masked[row, j] = E // R, -1
    args = (d["recv_topk_weights"], note4["recv_gbl_rank_prefix_sum"], note4["num_recv_tokens_per_expert"], E)
    gb = o.group_by_expert(d["recv_x"], ridx_bad, *args)
    gm = o.group_by_expert(d["recv_x"], ridx_masked, *args)
    if gb["status"] != _oracle.BAD_TOPK_IDX or gm["status"] != 0:
        errs.append(f"grouping status {gb['status']} / {gm['status']}, want the bad-id bit / 0")
    for k in ("grouped_x", "grouped_row", "slot_pos"):
        if not np.array_equal(gb[k], gm[k]):
            errs.append(f"grouping: a bad local id not skipped ({k})")
    # the grouping's outputs (rows, scales, row indices, weights, padding included) do not depend on what the
    # output buffers held: the same call with buffers full of stale values
    xs = rng.standard_normal((d["recv_x"].shape[0], 3)).astype(np.float32)
    fresh = o.group_by_expert(d["recv_x"], ridx_masked, *args, recv_x_scales=xs)
    m = fresh["num_grouped_rows"]
    rx = np.ascontiguousarray(d["recv_x"])
    gx = np.full((m, H), 0xABAB, np.uint16)
    gs = np.full((m, 3), 7.0, np.float32)
    grow = np.full(m, 99, np.int32)
    gw = np.full(m, 9.0, np.float32)
    pos = np.full(ridx.shape, 77, np.int32)
    mm = np.zeros(1, np.int32)
    idx_c = np.ascontiguousarray(ridx_masked, dtype=np.int64)
    w_c = np.ascontiguousarray(d["recv_topk_weights"], dtype=np.float32)
    gbl = np.ascontiguousarray(note4["recv_gbl_rank_prefix_sum"], dtype=np.int32)
    al = np.ascontiguousarray(note4["num_recv_tokens_per_expert"], dtype=np.int32)
    o.lib.oracle_group_by_expert(E, R, K, H * 2, p(rx), p(xs), 3, p(idx_c), p(w_c), p(gbl), p(al), rx.shape[0], m,
                                 p(gx), p(gs), p(grow), p(gw), p(pos), p(mm))
    for k, got in (("grouped_x", gx), ("grouped_x_scales", gs), ("grouped_row", grow), ("grouped_weights", gw),
                   ("slot_pos", pos)):
        if not np.array_equal(got, fresh[k]):
            errs.append(f"grouping: {k} depends on what the output buffer held")
    return errs
