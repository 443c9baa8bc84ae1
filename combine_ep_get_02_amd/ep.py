"""Thin Python binding of libep.so (the C ABI in include/ep.h).

The functions carry the C names and only marshal arguments: torch tensors
become raw device pointers, the stream defaults to torch's current stream,
and a non-OK status becomes an ``EpError``.  All computation happens in the
library's HIP kernels; there is no fallback path.  Torch is used for device
memory and streams only.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(_PKG, "libep.so")

EP_OK, EP_ERR_INVALID_ARG, EP_ERR_UNSUPPORTED, EP_ERR_HIP = 0, 1, 2, 3
EP_DEV_BAD_TOPK_IDX, EP_DEV_RECV_OVERFLOW, EP_DEV_COUNT_MISMATCH, EP_DEV_BAD_SEND_SLOT = 1, 2, 4, 8
EP_DEV_STALE_WORKSPACE = 16
EP_FORM_AUTO, EP_FORM_PUSH, EP_FORM_PULL = 0, 1, 2

EXPORTED = ("ep_get_layout", "ep_get_layout_noalloc", "ep_notify", "ep_layout_notify", "ep_dispatch", "ep_dispatch_fp8",
            "ep_dispatch_to_fp8", "ep_quantize_fp8", "ep_dequantize_fp8", "ep_dispatch_cached",
            "ep_dispatch_cached_to_fp8", "ep_group_by_expert", "ep_dispatch_grouped",
            "ep_combine", "ep_workspace_bytes", "ep_status_string")


class EpError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {ep_status_string(status)}")


class ep_shape_t(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int32) for name in (
        "num_tokens", "hidden", "num_topk", "num_experts", "num_ranks", "num_channels", "my_rank",
        "expert_alignment")]


_P = ctypes.c_void_p
_S = ctypes.POINTER(ep_shape_t)
_lib: ctypes.CDLL | None = None


def load(path: str = LIBRARY) -> ctypes.CDLL:
    """Load libep.so.  A missing library is an error: there is no fallback."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libep.so not built at {path}; run `python -m combine_ep_get_02_amd.build`")
    lib = ctypes.CDLL(path)
    lib.ep_get_layout.argtypes = [_S, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P, _P]
    lib.ep_get_layout_noalloc.argtypes = [_S, _P, _P, _P, _P, _P, _P, _P]
    lib.ep_notify.argtypes = [_S] + [_P] * 11 + [_P, ctypes.c_size_t, _P, _P]
    lib.ep_layout_notify.argtypes = [_S] + [_P] * 13 + [ctypes.c_size_t, _P, _P]
    lib.ep_dispatch.argtypes = [_S, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, ctypes.c_int32] + [_P] * 5 + \
        [ctypes.c_int32, _P, _P]
    lib.ep_dispatch_fp8.argtypes = [_S, _P, _P, ctypes.c_int32, _P, _P, _P, _P, _P, _P, ctypes.c_size_t,
                                    ctypes.c_int32] + [_P] * 6 + [ctypes.c_int32, _P, _P]
    lib.ep_dispatch_cached.argtypes = [_S, _P, ctypes.c_int32, _P, ctypes.c_int32, _P, ctypes.c_int32, _P, _P,
                                       ctypes.c_int32, _P, _P]
    lib.ep_group_by_expert.argtypes = [_S, _P, ctypes.c_int32, _P, ctypes.c_int32, _P, _P, _P, _P, ctypes.c_int32,
                                       ctypes.c_int32] + [_P] * 8
    lib.ep_dispatch_grouped.argtypes = [_S, _P, ctypes.c_int32, _P, ctypes.c_int32, _P, _P, _P, _P, _P, _P, _P,
                                        ctypes.c_size_t, ctypes.c_int32, _P, _P, _P, _P, ctypes.c_int32] + [_P] * 8
    lib.ep_combine.argtypes = [_S, _P, _P, _P, ctypes.c_int32, _P, _P, _P, _P]
    lib.ep_dispatch_to_fp8.argtypes = [_S, _P, ctypes.c_int32, _P, _P, _P, _P, _P, _P, ctypes.c_size_t,
                                       ctypes.c_int32] + [_P] * 8
    lib.ep_dispatch_cached_to_fp8.argtypes = [_S, _P, ctypes.c_int32, _P, ctypes.c_int32, _P, _P, _P, _P]
    lib.ep_quantize_fp8.argtypes = [_P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, _P, _P, _P]
    lib.ep_dequantize_fp8.argtypes = [_P, _P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, _P, _P]
    for name in ("ep_get_layout", "ep_get_layout_noalloc", "ep_notify", "ep_layout_notify", "ep_dispatch", "ep_dispatch_fp8", "ep_dispatch_cached",
                 "ep_group_by_expert", "ep_dispatch_grouped", "ep_combine", "ep_quantize_fp8", "ep_dequantize_fp8",
                 "ep_dispatch_to_fp8", "ep_dispatch_cached_to_fp8"):
        getattr(lib, name).restype = ctypes.c_int
    lib.ep_workspace_bytes.argtypes = [_S]
    lib.ep_workspace_bytes.restype = ctypes.c_size_t
    lib.ep_status_string.argtypes = [ctypes.c_int]
    lib.ep_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, where: str) -> None:
    if status != EP_OK:
        raise EpError(status, where)


def make_shape(num_tokens, hidden, num_topk, num_experts, num_ranks, num_channels, my_rank=0,
               expert_alignment=1) -> ep_shape_t:
    return ep_shape_t(num_tokens, hidden, num_topk, num_experts, num_ranks, num_channels, my_rank,
                      expert_alignment)


def ep_status_string(status: int) -> str:
    return load().ep_status_string(status).decode()


def ep_workspace_bytes(shape: ep_shape_t) -> int:
    return int(load().ep_workspace_bytes(ctypes.byref(shape)))


def ep_get_layout(shape, topk_idx, num_tokens_per_rank, num_tokens_per_rdma_rank, num_tokens_per_expert,
                  is_token_in_rank, workspace, dev_status=None, stream=None) -> None:
    _check(load().ep_get_layout(ctypes.byref(shape), _ptr(topk_idx), _ptr(num_tokens_per_rank),
                                _ptr(num_tokens_per_rdma_rank), _ptr(num_tokens_per_expert),
                                _ptr(is_token_in_rank), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                _ptr(dev_status), _stream(stream)), "ep_get_layout")


def ep_get_layout_noalloc(shape, topk_idx, num_tokens_per_rank, num_tokens_per_rdma_rank, num_tokens_per_expert,
                          is_token_in_rank, dev_status=None, stream=None) -> None:
    """ep_get_layout on the library's static scratch: no workspace, nothing allocated."""
    _check(load().ep_get_layout_noalloc(ctypes.byref(shape), _ptr(topk_idx), _ptr(num_tokens_per_rank),
                                        _ptr(num_tokens_per_rdma_rank), _ptr(num_tokens_per_expert),
                                        _ptr(is_token_in_rank), _ptr(dev_status), _stream(stream)),
           "ep_get_layout_noalloc")


def ep_notify(shape, is_token_in_rank, num_tokens_per_rank, num_tokens_per_rdma_rank, num_tokens_per_expert,
              gbl_channel_prefix_matrix, rdma_channel_prefix_matrix, recv_gbl_rank_prefix_sum,
              recv_rdma_rank_prefix_sum, num_recv_tokens_per_expert, num_recv_tokens, workspace,
              read_back: bool = False, dev_status=None, stream=None) -> int | None:
    """Returns N (host int) when ``read_back`` is set; the call then waits for the stream."""
    host = ctypes.c_int32(-1)
    _check(load().ep_notify(ctypes.byref(shape), _ptr(is_token_in_rank), _ptr(num_tokens_per_rank),
                            _ptr(num_tokens_per_rdma_rank), _ptr(num_tokens_per_expert),
                            _ptr(gbl_channel_prefix_matrix), _ptr(rdma_channel_prefix_matrix),
                            _ptr(recv_gbl_rank_prefix_sum), _ptr(recv_rdma_rank_prefix_sum),
                            _ptr(num_recv_tokens_per_expert), _ptr(num_recv_tokens),
                            ctypes.addressof(host) if read_back else None, _ptr(workspace),
                            workspace.numel() * workspace.element_size(), _ptr(dev_status), _stream(stream)),
           "ep_notify")
    return int(host.value) if read_back else None


def _ws(workspace):
    """Pointer and size of an optional workspace tensor."""
    if workspace is None:
        return None, 0
    return _ptr(workspace), workspace.numel() * workspace.element_size()


def ep_layout_notify(shape, topk_idx, num_tokens_per_rank, num_tokens_per_rdma_rank, num_tokens_per_expert,
                     is_token_in_rank, gbl_channel_prefix_matrix, rdma_channel_prefix_matrix, recv_gbl_rank_prefix_sum,
                     recv_rdma_rank_prefix_sum, num_recv_tokens_per_expert, num_recv_tokens, workspace,
                     read_back: bool = False, dev_status=None, stream=None) -> int | None:
    """ep_get_layout and ep_notify in one launch.  Returns N (host int) when ``read_back``
    is set; the call then waits for the stream."""
    host = ctypes.c_int32(-1)
    _check(load().ep_layout_notify(ctypes.byref(shape), _ptr(topk_idx), _ptr(num_tokens_per_rank),
                                   _ptr(num_tokens_per_rdma_rank), _ptr(num_tokens_per_expert),
                                   _ptr(is_token_in_rank), _ptr(gbl_channel_prefix_matrix),
                                   _ptr(rdma_channel_prefix_matrix), _ptr(recv_gbl_rank_prefix_sum),
                                   _ptr(recv_rdma_rank_prefix_sum), _ptr(num_recv_tokens_per_expert),
                                   _ptr(num_recv_tokens), ctypes.addressof(host) if read_back else None,
                                   _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(dev_status),
                                   _stream(stream)), "ep_layout_notify")
    return int(host.value) if read_back else None


def ep_dispatch(shape, x, topk_idx, topk_weights, is_token_in_rank, gbl_channel_prefix_matrix,
                recv_gbl_rank_prefix_sum, workspace, recv_capacity, recv_x, recv_topk_weights, recv_topk_idx,
                recv_src_info, send_slot, dev_status=None, stream=None, form=EP_FORM_AUTO) -> None:
    """workspace: the one ep_notify filled for this is_token_in_rank, or None (the routing is
    then worked out from is_token_in_rank and the prefix sums inside the call).  form: an
    EP_FORM_* value (push when x is only in HBM, pull when it was just written)."""
    ws, ws_bytes = _ws(workspace)
    _check(load().ep_dispatch(ctypes.byref(shape), _ptr(x), _ptr(topk_idx), _ptr(topk_weights),
                              _ptr(is_token_in_rank), _ptr(gbl_channel_prefix_matrix),
                              _ptr(recv_gbl_rank_prefix_sum), ws, ws_bytes, int(recv_capacity), _ptr(recv_x),
                              _ptr(recv_topk_weights), _ptr(recv_topk_idx), _ptr(recv_src_info), _ptr(send_slot),
                              int(form), _ptr(dev_status), _stream(stream)), "ep_dispatch")


def ep_dispatch_fp8(shape, x, x_scales, num_scales, topk_idx, topk_weights, is_token_in_rank,
                    gbl_channel_prefix_matrix, recv_gbl_rank_prefix_sum, workspace, recv_capacity, recv_x,
                    recv_x_scales, recv_topk_weights, recv_topk_idx, recv_src_info, send_slot, dev_status=None,
                    stream=None, form=EP_FORM_AUTO) -> None:
    ws, ws_bytes = _ws(workspace)
    _check(load().ep_dispatch_fp8(ctypes.byref(shape), _ptr(x), _ptr(x_scales), int(num_scales), _ptr(topk_idx),
                                  _ptr(topk_weights), _ptr(is_token_in_rank), _ptr(gbl_channel_prefix_matrix),
                                  _ptr(recv_gbl_rank_prefix_sum), ws, ws_bytes, int(recv_capacity), _ptr(recv_x),
                                  _ptr(recv_x_scales), _ptr(recv_topk_weights), _ptr(recv_topk_idx),
                                  _ptr(recv_src_info), _ptr(send_slot), int(form), _ptr(dev_status),
                                  _stream(stream)), "ep_dispatch_fp8")


def ep_dispatch_cached(shape, x, elem_bytes, x_scales, num_scales, send_slot, recv_capacity, recv_x,
                       recv_x_scales=None, dev_status=None, stream=None, form=EP_FORM_AUTO) -> None:
    _check(load().ep_dispatch_cached(ctypes.byref(shape), _ptr(x), int(elem_bytes), _ptr(x_scales), int(num_scales),
                                     _ptr(send_slot), int(recv_capacity), _ptr(recv_x), _ptr(recv_x_scales),
                                     int(form), _ptr(dev_status), _stream(stream)), "ep_dispatch_cached")


def ep_group_by_expert(shape, recv_x, elem_bytes, recv_x_scales, num_scales, recv_topk_idx, recv_topk_weights,
                       recv_gbl_rank_prefix_sum, num_recv_tokens_per_expert, num_recv_rows, grouped_capacity,
                       grouped_x, grouped_x_scales, grouped_row, grouped_weights, slot_pos, num_grouped_rows,
                       dev_status=None, stream=None) -> None:
    _check(load().ep_group_by_expert(ctypes.byref(shape), _ptr(recv_x), int(elem_bytes), _ptr(recv_x_scales),
                                     int(num_scales), _ptr(recv_topk_idx), _ptr(recv_topk_weights),
                                     _ptr(recv_gbl_rank_prefix_sum), _ptr(num_recv_tokens_per_expert),
                                     int(num_recv_rows), int(grouped_capacity), _ptr(grouped_x),
                                     _ptr(grouped_x_scales), _ptr(grouped_row), _ptr(grouped_weights), _ptr(slot_pos),
                                     _ptr(num_grouped_rows), _ptr(dev_status), _stream(stream)),
           "ep_group_by_expert")


def ep_dispatch_grouped(shape, x, elem_bytes, x_scales, num_scales, topk_idx, topk_weights, is_token_in_rank,
                        gbl_channel_prefix_matrix, recv_gbl_rank_prefix_sum, num_recv_tokens_per_expert, workspace,
                        recv_capacity, recv_topk_weights, recv_topk_idx, recv_src_info, send_slot, grouped_capacity,
                        grouped_x, grouped_x_scales, grouped_row, grouped_weights, slot_pos, num_grouped_rows,
                        dev_status=None, stream=None) -> None:
    ws, ws_bytes = _ws(workspace)
    _check(load().ep_dispatch_grouped(ctypes.byref(shape), _ptr(x), int(elem_bytes), _ptr(x_scales), int(num_scales),
                                      _ptr(topk_idx), _ptr(topk_weights), _ptr(is_token_in_rank),
                                      _ptr(gbl_channel_prefix_matrix), _ptr(recv_gbl_rank_prefix_sum),
                                      _ptr(num_recv_tokens_per_expert), ws, ws_bytes, int(recv_capacity),
                                      _ptr(recv_topk_weights), _ptr(recv_topk_idx), _ptr(recv_src_info),
                                      _ptr(send_slot), int(grouped_capacity), _ptr(grouped_x), _ptr(grouped_x_scales),
                                      _ptr(grouped_row), _ptr(grouped_weights), _ptr(slot_pos),
                                      _ptr(num_grouped_rows), _ptr(dev_status), _stream(stream)),
           "ep_dispatch_grouped")


def ep_combine(shape, y, recv_topk_weights, send_slot, num_recv_rows, combined_x, combined_topk_weights=None,
               dev_status=None, stream=None) -> None:
    _check(load().ep_combine(ctypes.byref(shape), _ptr(y), _ptr(recv_topk_weights), _ptr(send_slot),
                             int(num_recv_rows), _ptr(combined_x), _ptr(combined_topk_weights), _ptr(dev_status),
                             _stream(stream)), "ep_combine")


def ep_dispatch_to_fp8(shape, x, num_scales, topk_idx, topk_weights, is_token_in_rank, gbl_channel_prefix_matrix,
                       recv_gbl_rank_prefix_sum, workspace, recv_capacity, recv_x, recv_x_scales, recv_topk_weights,
                       recv_topk_idx, recv_src_info, send_slot, dev_status=None, stream=None) -> None:
    ws, ws_bytes = _ws(workspace)
    _check(load().ep_dispatch_to_fp8(ctypes.byref(shape), _ptr(x), int(num_scales), _ptr(topk_idx), _ptr(topk_weights),
                                     _ptr(is_token_in_rank), _ptr(gbl_channel_prefix_matrix),
                                     _ptr(recv_gbl_rank_prefix_sum), ws, ws_bytes, int(recv_capacity), _ptr(recv_x),
                                     _ptr(recv_x_scales), _ptr(recv_topk_weights), _ptr(recv_topk_idx),
                                     _ptr(recv_src_info), _ptr(send_slot), _ptr(dev_status), _stream(stream)),
           "ep_dispatch_to_fp8")


def ep_dispatch_cached_to_fp8(shape, x, num_scales, send_slot, recv_capacity, recv_x, recv_x_scales, dev_status=None,
                              stream=None) -> None:
    _check(load().ep_dispatch_cached_to_fp8(ctypes.byref(shape), _ptr(x), int(num_scales), _ptr(send_slot),
                                            int(recv_capacity), _ptr(recv_x), _ptr(recv_x_scales), _ptr(dev_status),
                                            _stream(stream)), "ep_dispatch_cached_to_fp8")


def ep_quantize_fp8(x, num_rows, hidden, num_scales, x_fp8, x_scales, stream=None) -> None:
    _check(load().ep_quantize_fp8(_ptr(x), int(num_rows), int(hidden), int(num_scales), _ptr(x_fp8), _ptr(x_scales),
                                  _stream(stream)), "ep_quantize_fp8")


def ep_dequantize_fp8(x_fp8, x_scales, num_rows, hidden, num_scales, out, stream=None) -> None:
    _check(load().ep_dequantize_fp8(_ptr(x_fp8), _ptr(x_scales), int(num_rows), int(hidden), int(num_scales),
                                    _ptr(out), _stream(stream)), "ep_dequantize_fp8")


# ----------------------------------------------------------------------------- buffers
@dataclass
class Buffers:
    """Every device buffer of one pass, allocated by torch for a shape."""
    shape: ep_shape_t
    capacity: int
    per_rank: torch.Tensor
    per_node: torch.Tensor
    per_expert: torch.Tensor
    in_rank: torch.Tensor
    gbl: torch.Tensor
    rdma: torch.Tensor
    recv_gbl: torch.Tensor
    recv_rdma: torch.Tensor
    recv_per_expert: torch.Tensor
    num_recv: torch.Tensor
    workspace: torch.Tensor
    recv_x: torch.Tensor
    recv_w: torch.Tensor
    recv_idx: torch.Tensor | None
    src_info: torch.Tensor
    send_slot: torch.Tensor
    combined_x: torch.Tensor
    combined_w: torch.Tensor
    dev_status: torch.Tensor


def allocate(shape: ep_shape_t, capacity: int, device="cuda", with_recv_idx: bool = True) -> Buffers:
    T, H, K = shape.num_tokens, shape.hidden, shape.num_topk
    R, E, C = shape.num_ranks, shape.num_experts, shape.num_channels
    nodes = max(1, R // 8)
    i32 = dict(dtype=torch.int32, device=device)
    cap = max(int(capacity), 0)
    return Buffers(
        shape=shape, capacity=cap,
        per_rank=torch.empty(R, **i32), per_node=torch.empty(nodes, **i32), per_expert=torch.empty(E, **i32),
        in_rank=torch.empty((T, R), dtype=torch.uint8, device=device),
        gbl=torch.empty((R, C), **i32), rdma=torch.empty((nodes, C), **i32), recv_gbl=torch.empty(R, **i32),
        recv_rdma=torch.empty(nodes, **i32), recv_per_expert=torch.empty(E, **i32), num_recv=torch.empty(1, **i32),
        workspace=torch.zeros(max(ep_workspace_bytes(shape), 256), dtype=torch.uint8, device=device),
        recv_x=torch.empty((cap, H), dtype=torch.bfloat16, device=device),
        recv_w=torch.empty((cap, K), dtype=torch.float32, device=device),
        recv_idx=torch.empty((cap, K), dtype=torch.int64, device=device) if with_recv_idx else None,
        src_info=torch.empty((cap, 2), **i32), send_slot=torch.empty((T, R), **i32),
        combined_x=torch.empty((T, H), dtype=torch.bfloat16, device=device),
        combined_w=torch.empty((T, K), dtype=torch.float32, device=device),
        dev_status=torch.zeros(1, **i32))


def run_layout(b: Buffers, topk_idx, stream=None) -> None:
    ep_get_layout(b.shape, topk_idx, b.per_rank, b.per_node, b.per_expert, b.in_rank, b.workspace, b.dev_status,
                  stream)


def run_notify(b: Buffers, read_back: bool = False, stream=None) -> int | None:
    return ep_notify(b.shape, b.in_rank, b.per_rank, b.per_node, b.per_expert, b.gbl, b.rdma, b.recv_gbl,
                     b.recv_rdma, b.recv_per_expert, b.num_recv, b.workspace, read_back, b.dev_status, stream)


def run_layout_notify(b: Buffers, topk_idx, read_back: bool = False, stream=None) -> int | None:
    return ep_layout_notify(b.shape, topk_idx, b.per_rank, b.per_node, b.per_expert, b.in_rank, b.gbl, b.rdma,
                            b.recv_gbl, b.recv_rdma, b.recv_per_expert, b.num_recv, b.workspace, read_back,
                            b.dev_status, stream)


def run_dispatch(b: Buffers, x, topk_idx, topk_weights, use_workspace: bool = True, stream=None,
                 form=EP_FORM_AUTO) -> None:
    """use_workspace: take the routing state notify left in b.workspace; False: work it
    out from b.in_rank and the prefix sums inside the call."""
    ep_dispatch(b.shape, x, topk_idx, topk_weights, b.in_rank, b.gbl, b.recv_gbl,
                b.workspace if use_workspace else None, b.capacity, b.recv_x, b.recv_w, b.recv_idx, b.src_info,
                b.send_slot, b.dev_status, stream, form)


def run_combine(b: Buffers, y=None, num_recv_rows=None, with_weights: bool = True, stream=None) -> None:
    ep_combine(b.shape, b.recv_x if y is None else y, b.recv_w, b.send_slot,
               b.capacity if num_recv_rows is None else num_recv_rows, b.combined_x,
               b.combined_w if with_weights else None, b.dev_status, stream)


@dataclass
class GroupBuffers:
    """Outputs of the grouping by local expert for `capacity` grouped rows."""
    capacity: int
    grouped_x: torch.Tensor
    grouped_row: torch.Tensor
    grouped_w: torch.Tensor
    slot_pos: torch.Tensor
    num_grouped: torch.Tensor


def allocate_group(b: Buffers, capacity: int, device="cuda") -> GroupBuffers:
    """capacity: grouped rows, normally the sum of b.recv_per_expert after notify."""
    cap = max(int(capacity), 0)
    i32 = dict(dtype=torch.int32, device=device)
    return GroupBuffers(capacity=cap,
                        grouped_x=torch.empty((cap, b.shape.hidden), dtype=torch.bfloat16, device=device),
                        grouped_row=torch.empty(cap, **i32), grouped_w=torch.empty(cap, dtype=torch.float32, device=device),
                        slot_pos=torch.empty((b.capacity, b.shape.num_topk), **i32), num_grouped=torch.empty(1, **i32))


def run_group(b: Buffers, g: GroupBuffers, num_recv_rows=None, stream=None) -> None:
    ep_group_by_expert(b.shape, b.recv_x, 2, None, 0, b.recv_idx, b.recv_w, b.recv_gbl, b.recv_per_expert,
                       b.capacity if num_recv_rows is None else num_recv_rows, g.capacity, g.grouped_x, None,
                       g.grouped_row, g.grouped_w, g.slot_pos, g.num_grouped, b.dev_status, stream)


def run_dispatch_grouped(b: Buffers, g: GroupBuffers, x, topk_idx, topk_weights, stream=None) -> None:
    """Dispatch of bf16 rows straight into g's grouped layout (b.recv_x is neither written nor read)."""
    ep_dispatch_grouped(b.shape, x, 2, None, 0, topk_idx, topk_weights, b.in_rank, b.gbl, b.recv_gbl,
                        b.recv_per_expert, b.workspace,
                        b.capacity, b.recv_w, b.recv_idx, b.src_info, b.send_slot, g.capacity, g.grouped_x, None,
                        g.grouped_row, g.grouped_w, g.slot_pos, g.num_grouped, b.dev_status, stream)
