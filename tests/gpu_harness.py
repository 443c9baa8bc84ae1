"""Runs the HIP path through the C ABI and the oracle side by side on the same
seeded inputs, and returns both sides' outputs as numpy arrays."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from combine_ep_get_02_amd import ep

SENTINEL_I32 = -777


def to_dev_bf16(u16: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).cuda().view(torch.bfloat16)


def bf16_host(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def random_rows(rng: np.random.Generator, n: int, h: int) -> np.ndarray:
    """bf16 bit patterns of random sign, exponent in [2^-6, 2^5], random mantissa."""
    bits = rng.integers(0, 1 << 16, size=(n, h), dtype=np.uint16)
    exp = ((bits >> 7) % 12 + 121).astype(np.uint16)
    return (bits & np.uint16(0x807F)) | (exp << np.uint16(7))


def run_both(x, topk_idx, topk_weights, E, R, C, my_rank=0, align=1, capacity=None, y=None, orc=None,
             in_rank_override=None, with_recv_idx=True):
    """All four stages on the GPU (through the C ABI) and in the oracle."""
    orc = orc or oracle.Oracle()
    T, H = x.shape
    K = topk_idx.shape[1]
    shape = ep.make_shape(T, H, K, E, R, C, my_rank, align)
    cap = capacity if capacity is not None else T * min(R, K)

    b = ep.allocate(shape, cap, with_recv_idx=with_recv_idx)
    for t in (b.gbl, b.rdma, b.recv_gbl, b.recv_rdma, b.recv_per_expert, b.num_recv, b.send_slot, b.src_info):
        t.fill_(SENTINEL_I32)
    b.recv_w.fill_(-3.0)
    # receive rows poisoned with all-ones bytes (a NaN pattern in bf16): a row dispatch
    # fails to write cannot match the oracle's row by accident
    b.recv_x.view(torch.int16).fill_(-1)
    if b.recv_idx is not None:
        b.recv_idx.fill_(-777)
    b.combined_w.fill_(-3.0)

    dx = to_dev_bf16(x)
    didx = torch.from_numpy(np.ascontiguousarray(topk_idx, dtype=np.int64)).cuda()
    dw = torch.from_numpy(np.ascontiguousarray(topk_weights, dtype=np.float32)).cuda()

    ep.run_layout(b, didx)
    if in_rank_override is not None:
        b.in_rank.copy_(torch.from_numpy(in_rank_override))
    n_host = ep.run_notify(b, read_back=True)
    ep.run_dispatch(b, dx, didx, dw)
    torch.cuda.synchronize()
    gpu = dict(
        num_tokens_per_rank=b.per_rank.cpu().numpy(), num_tokens_per_rdma_rank=b.per_node.cpu().numpy(),
        num_tokens_per_expert=b.per_expert.cpu().numpy(), is_token_in_rank=b.in_rank.cpu().numpy(),
        gbl_channel_prefix_matrix=b.gbl.cpu().numpy(), rdma_channel_prefix_matrix=b.rdma.cpu().numpy(),
        recv_gbl_rank_prefix_sum=b.recv_gbl.cpu().numpy(), recv_rdma_rank_prefix_sum=b.recv_rdma.cpu().numpy(),
        num_recv_tokens_per_expert=b.recv_per_expert.cpu().numpy(), num_recv_tokens=int(b.num_recv.item()),
        num_recv_host=n_host, send_slot=b.send_slot.cpu().numpy())
    n = gpu["num_recv_tokens"]
    rows = min(n, cap)
    gpu["recv_x"] = bf16_host(b.recv_x[:rows])
    gpu["recv_topk_weights"] = b.recv_w[:rows].cpu().numpy()
    gpu["recv_topk_idx"] = b.recv_idx[:rows].cpu().numpy() if b.recv_idx is not None else None
    gpu["recv_src_info"] = b.src_info[:rows].cpu().numpy()

    # combine on identity experts, then on independent expert outputs y
    ep.run_combine(b, num_recv_rows=rows)
    torch.cuda.synchronize()
    gpu["combined_x"] = bf16_host(b.combined_x)
    gpu["combined_topk_weights"] = b.combined_w.cpu().numpy()
    if y is not None:
        dy = to_dev_bf16(y)
        ep.run_combine(b, y=dy, num_recv_rows=y.shape[0])
        torch.cuda.synchronize()
        gpu["combined_x_y"] = bf16_host(b.combined_x)
    gpu["dev_status"] = int(b.dev_status.item())

    # oracle on the same inputs
    lay = orc.layout(topk_idx, E, R)
    in_rank = lay["is_token_in_rank"] if in_rank_override is None else (in_rank_override != 0).astype(np.uint8)
    note = orc.notify(in_rank, lay["num_tokens_per_rank"], lay["num_tokens_per_rdma_rank"],
                      lay["num_tokens_per_expert"], C, align)
    dis = orc.dispatch(x, topk_idx, topk_weights, in_rank, note["gbl_channel_prefix_matrix"],
                       note["recv_gbl_rank_prefix_sum"], E, my_rank, recv_capacity=cap,
                       with_topk_idx=with_recv_idx)
    com = orc.combine(dis["recv_x"][:rows], dis["recv_topk_weights"][:rows], dis["send_slot"], rows)
    ref = dict(lay)
    ref.update(note)
    ref.update(dis)
    ref["recv_x"] = dis["recv_x"][:rows]
    ref["recv_topk_weights"] = dis["recv_topk_weights"][:rows]
    ref["recv_topk_idx"] = dis["recv_topk_idx"][:rows] if dis["recv_topk_idx"] is not None else None
    ref["recv_src_info"] = dis["recv_src_info"][:rows]
    ref["combined_x"] = com["combined_x"]
    ref["combined_topk_weights"] = com["combined_topk_weights"]
    # the same weighted sums in binary64, for the secondary bound on the bf16 outputs
    ref["combined_x_f64"] = orc.combine_f64(dis["recv_x"][:rows], dis["recv_topk_weights"][:rows], dis["send_slot"],
                                            rows)[0]
    if y is not None:
        ref["combined_x_y"] = orc.combine(y, dis["recv_topk_weights"][:rows], dis["send_slot"], y.shape[0])["combined_x"]
        ref["combined_x_y_f64"] = orc.combine_f64(y, dis["recv_topk_weights"][:rows], dis["send_slot"],
                                                  y.shape[0])[0]
    ref["status"] = lay["status"] | note["status"] | dis["status"] | com["status"]
    return gpu, ref


EXACT_KEYS = ("num_tokens_per_rank", "num_tokens_per_rdma_rank", "num_tokens_per_expert", "is_token_in_rank",
              "gbl_channel_prefix_matrix", "rdma_channel_prefix_matrix", "recv_gbl_rank_prefix_sum",
              "recv_rdma_rank_prefix_sum", "num_recv_tokens_per_expert", "num_recv_tokens", "send_slot",
              "recv_x", "recv_topk_weights", "recv_topk_idx", "recv_src_info", "combined_topk_weights")


def compare(gpu: dict, ref: dict, tol: float = 1e-2) -> list[str]:
    """Integer, index and copied data: bit-exact.  Combined rows: max |diff| <= tol
    (the bar for bf16 outputs with fp32 accumulation), and the count of
    differing elements is reported."""
    errs = []
    for k in EXACT_KEYS:
        g, r = gpu.get(k), ref.get(k)
        if g is None and r is None:
            continue
        g, r = np.asarray(g), np.asarray(r)
        if g.shape != r.shape:
            errs.append(f"{k}: shape {g.shape} vs {r.shape}")
        elif g.dtype.kind == "f":
            if not np.array_equal(g.view(np.uint32), r.view(np.uint32)):
                errs.append(f"{k}: {int((g.view(np.uint32) != r.view(np.uint32)).sum())} bit differences")
        elif not np.array_equal(g, r):
            errs.append(f"{k}: {int((g != r).sum())} differences")
    if gpu.get("num_recv_host") is not None and gpu["num_recv_host"] != ref["num_recv_tokens"]:
        errs.append("host copy of N differs")
    for k in ("combined_x", "combined_x_y"):
        if k not in gpu:
            continue
        g = (gpu[k].astype(np.uint32) << 16).view(np.float32)
        r = (ref[k].astype(np.uint32) << 16).view(np.float32)
        d = np.abs(g.astype(np.float64) - r.astype(np.float64))
        if d.size and d.max() > tol:
            errs.append(f"{k}: max |diff| {d.max():.4g} > {tol}")
        # secondary bound against the binary64 sum: max(tol, one bf16 ulp of the
        # exact value), the most a correctly rounded fp32 chain can be off after
        # its final rounding to bf16
        f = ref.get(k + "_f64")
        if f is not None and f.size:
            lim = np.maximum(tol, bf16_ulp(f))
            e = np.abs(g.astype(np.float64) - f)
            if np.any(e > lim):
                errs.append(f"{k}: {int((e > lim).sum())} elements beyond max({tol}, ulp_bf16) of the binary64 sum")
    return errs


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |v| (8 significant bits); the subnormal spacing at 0."""
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, 2.0 ** (e - 7), 2.0 ** -133)


def combine_bit_differences(gpu: dict, ref: dict) -> dict:
    """Elements of the combined rows whose bf16 bits differ.  Both sides use the
    same reduction order and fp32 fma, so zero is expected; this is stricter
    than the tolerance bar."""
    return {k: int((gpu[k] != ref[k]).sum()) for k in ("combined_x", "combined_x_y") if k in gpu}
