"""CPU oracle for the expert-parallel dispatch/combine core.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path never does.  It
wraps ``ep_oracle.c`` (plain single-threaded C, built with gcc) through ctypes
and numpy.  It shares no code with the HIP library.

Every function takes and returns numpy arrays; shapes follow the definitions
in ``ep_oracle.c`` (each cites the page passage it follows).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "ep_oracle.c")
LIBRARY = os.path.join(_HERE, "libep_oracle.so")
CFLAGS = ["-O2", "-ffp-contract=off", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra"]

BAD_TOPK_IDX = 1
RECV_OVERFLOW = 2
COUNT_MISMATCH = 4
BAD_SEND_SLOT = 8


def build(source: str = SOURCE, out: str = LIBRARY) -> str:
    """Compile the oracle with gcc; returns the path of the shared library."""
    cmd = ["gcc", *CFLAGS, source, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


_P = ctypes.c_void_p
_I = ctypes.c_int32
_L = ctypes.c_int64


def _declare(lib: ctypes.CDLL) -> ctypes.CDLL:
    lib.oracle_layout.argtypes = [_I, _I, _I, _I, _P, _P, _P, _P, _P]
    lib.oracle_notify.argtypes = [_I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]
    lib.oracle_dispatch.argtypes = [_I, _I, _I, _I, _I, _I, _I, _I] + [_P] * 11
    lib.oracle_combine.argtypes = [_I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P]
    lib.oracle_combine_f64.argtypes = [_I, _I, _I, _I, _I, _P, _P, _P, _P]
    lib.oracle_dispatch_fp8.argtypes = [_I, _I, _I, _I, _I, _I, _I, _I, _P, _P, _I] + [_P] * 11
    lib.oracle_dispatch_cached.argtypes = [_I, _I, _L, _P, _P, _I, _P, _I, _P, _P]
    lib.oracle_group_by_expert.argtypes = [_I, _I, _I, _L, _P, _P, _I, _P, _P, _P, _P, _I, _I] + [_P] * 6
    lib.oracle_bf16_round.argtypes = [_P, _P, _L]
    lib.oracle_e4m3_encode.argtypes = [_P, _P, _L]
    lib.oracle_e4m3_decode.argtypes = [_P, _P, _L]
    lib.oracle_quantize_e4m3.argtypes = [_L, _I, _I, _P, _P, _P]
    lib.oracle_dequantize_e4m3.argtypes = [_L, _I, _I, _P, _P, _P]
    for name in ("oracle_layout", "oracle_notify", "oracle_dispatch", "oracle_combine", "oracle_combine_f64",
                 "oracle_dispatch_fp8", "oracle_dispatch_cached", "oracle_quantize_e4m3", "oracle_dequantize_e4m3"):
        getattr(lib, name).restype = ctypes.c_int
    for name in ("oracle_bf16_round", "oracle_e4m3_encode", "oracle_e4m3_decode"):
        getattr(lib, name).restype = None
    return lib


def load(path: str = LIBRARY) -> ctypes.CDLL:
    """Load a built oracle library (building it first if it is absent)."""
    if not os.path.exists(path):
        build(out=path)
    return _declare(ctypes.CDLL(path))


_lib: ctypes.CDLL | None = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        _lib = load()
    return _lib


def _ptr(a: np.ndarray | None) -> int | None:
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def num_nodes(R: int) -> int:
    return max(1, R // 8)


class Oracle:
    """Numpy front end of one oracle library (the default one, or a variant)."""

    def __init__(self, handle: ctypes.CDLL | None = None):
        self.lib = handle if handle is not None else lib()

    def layout(self, topk_idx: np.ndarray, E: int, R: int):
        topk_idx = np.ascontiguousarray(topk_idx, dtype=np.int64)
        T, K = topk_idx.shape
        per_rank = np.zeros(R, np.int32)
        per_node = np.zeros(num_nodes(R), np.int32)
        per_expert = np.zeros(E, np.int32)
        in_rank = np.zeros((T, R), np.uint8)
        st = self.lib.oracle_layout(T, K, E, R, _ptr(topk_idx), _ptr(per_rank), _ptr(per_node),
                                    _ptr(per_expert), _ptr(in_rank))
        return dict(num_tokens_per_rank=per_rank, num_tokens_per_rdma_rank=per_node,
                    num_tokens_per_expert=per_expert, is_token_in_rank=in_rank, status=st)

    def notify(self, is_token_in_rank, num_tokens_per_rank, num_tokens_per_rdma_rank,
               num_tokens_per_expert, C: int, expert_alignment: int = 1):
        in_rank = np.ascontiguousarray(is_token_in_rank, dtype=np.uint8)
        T, R = in_rank.shape
        E = len(num_tokens_per_expert)
        nodes = num_nodes(R)
        gbl = np.zeros((R, C), np.int32)
        rdma = np.zeros((nodes, C), np.int32)
        recv_gbl = np.zeros(R, np.int32)
        recv_rdma = np.zeros(nodes, np.int32)
        recv_per_expert = np.zeros(E, np.int32)
        n_recv = np.zeros(1, np.int32)
        a = [np.ascontiguousarray(v, dtype=np.int32) for v in
             (num_tokens_per_rank, num_tokens_per_rdma_rank, num_tokens_per_expert)]
        st = self.lib.oracle_notify(T, E, R, C, expert_alignment, _ptr(in_rank), _ptr(a[0]), _ptr(a[1]),
                                    _ptr(a[2]), _ptr(gbl), _ptr(rdma), _ptr(recv_gbl), _ptr(recv_rdma),
                                    _ptr(recv_per_expert), _ptr(n_recv))
        return dict(gbl_channel_prefix_matrix=gbl, rdma_channel_prefix_matrix=rdma,
                    recv_gbl_rank_prefix_sum=recv_gbl, recv_rdma_rank_prefix_sum=recv_rdma,
                    num_recv_tokens_per_expert=recv_per_expert, num_recv_tokens=int(n_recv[0]), status=st)

    def dispatch(self, x, topk_idx, topk_weights, is_token_in_rank, gbl_channel_prefix_matrix,
                 recv_gbl_rank_prefix_sum, E: int, my_rank: int = 0, recv_capacity: int | None = None,
                 with_topk_idx: bool = True):
        x = np.ascontiguousarray(x, dtype=np.uint16)
        topk_idx = np.ascontiguousarray(topk_idx, dtype=np.int64)
        topk_weights = np.ascontiguousarray(topk_weights, dtype=np.float32)
        in_rank = np.ascontiguousarray(is_token_in_rank, dtype=np.uint8)
        gbl = np.ascontiguousarray(gbl_channel_prefix_matrix, dtype=np.int32)
        recv_gbl = np.ascontiguousarray(recv_gbl_rank_prefix_sum, dtype=np.int32)
        T, H = x.shape
        K = topk_idx.shape[1]
        R, C = gbl.shape
        n = int(recv_gbl[-1]) if R else 0
        cap = n if recv_capacity is None else recv_capacity
        recv_x = np.zeros((cap, H), np.uint16)
        recv_w = np.zeros((cap, K), np.float32)
        recv_idx = np.zeros((cap, K), np.int64) if with_topk_idx else None
        src_info = np.zeros((cap, 2), np.int32)
        send_slot = np.zeros((T, R), np.int32)
        st = self.lib.oracle_dispatch(T, H, K, E, R, C, my_rank, cap, _ptr(x), _ptr(topk_idx),
                                      _ptr(topk_weights), _ptr(in_rank), _ptr(gbl), _ptr(recv_gbl),
                                      _ptr(recv_x), _ptr(recv_w), _ptr(recv_idx), _ptr(src_info),
                                      _ptr(send_slot))
        return dict(recv_x=recv_x, recv_topk_weights=recv_w, recv_topk_idx=recv_idx,
                    recv_src_info=src_info, send_slot=send_slot, status=st)

    def dispatch_fp8(self, x8, x_scales, topk_idx, topk_weights, is_token_in_rank, gbl_channel_prefix_matrix,
                     recv_gbl_rank_prefix_sum, E: int, my_rank: int = 0, recv_capacity: int | None = None,
                     with_topk_idx: bool = True):
        """fp8 rows (uint8 bit patterns [t][h]) plus float scales [t][num_scales]."""
        x8 = np.ascontiguousarray(x8, dtype=np.uint8)
        x_scales = np.ascontiguousarray(x_scales, dtype=np.float32)
        topk_idx = np.ascontiguousarray(topk_idx, dtype=np.int64)
        topk_weights = np.ascontiguousarray(topk_weights, dtype=np.float32)
        in_rank = np.ascontiguousarray(is_token_in_rank, dtype=np.uint8)
        gbl = np.ascontiguousarray(gbl_channel_prefix_matrix, dtype=np.int32)
        recv_gbl = np.ascontiguousarray(recv_gbl_rank_prefix_sum, dtype=np.int32)
        T, H = x8.shape
        NS = x_scales.shape[1]
        K = topk_idx.shape[1]
        R, C = gbl.shape
        n = int(recv_gbl[-1]) if R else 0
        cap = n if recv_capacity is None else recv_capacity
        recv_x = np.zeros((cap, H), np.uint8)
        recv_s = np.zeros((cap, NS), np.float32)
        recv_w = np.zeros((cap, K), np.float32)
        recv_idx = np.zeros((cap, K), np.int64) if with_topk_idx else None
        src_info = np.zeros((cap, 2), np.int32)
        send_slot = np.zeros((T, R), np.int32)
        st = self.lib.oracle_dispatch_fp8(T, H, K, E, R, C, my_rank, cap, _ptr(x8), _ptr(x_scales), NS,
                                          _ptr(topk_idx), _ptr(topk_weights), _ptr(in_rank), _ptr(gbl),
                                          _ptr(recv_gbl), _ptr(recv_x), _ptr(recv_s), _ptr(recv_w), _ptr(recv_idx),
                                          _ptr(src_info), _ptr(send_slot))
        return dict(recv_x=recv_x, recv_x_scales=recv_s, recv_topk_weights=recv_w, recv_topk_idx=recv_idx,
                    recv_src_info=src_info, send_slot=send_slot, status=st)

    def dispatch_cached(self, x, send_slot, recv_capacity: int, x_scales=None):
        """Rows of any element type (moved as bytes) to the rows send_slot names."""
        x = np.ascontiguousarray(x)
        T = x.shape[0]
        row_bytes = int(np.prod(x.shape[1:], dtype=np.int64)) * x.itemsize
        send_slot = np.ascontiguousarray(send_slot, dtype=np.int32)
        R = send_slot.shape[1]
        NS = 0 if x_scales is None else x_scales.shape[1]
        xs = None if x_scales is None else np.ascontiguousarray(x_scales, dtype=np.float32)
        recv_x = np.zeros((recv_capacity,) + x.shape[1:], x.dtype)
        recv_s = np.zeros((recv_capacity, NS), np.float32) if NS else None
        st = self.lib.oracle_dispatch_cached(T, R, row_bytes, _ptr(x), _ptr(xs), NS, _ptr(send_slot),
                                             recv_capacity, _ptr(recv_x), _ptr(recv_s))
        return dict(recv_x=recv_x, recv_x_scales=recv_s, status=st)

    def group_by_expert(self, recv_x, recv_topk_idx, recv_topk_weights, recv_gbl_rank_prefix_sum,
                        aligned_per_expert, E: int, grouped_capacity: int | None = None, recv_x_scales=None,
                        num_recv_rows: int | None = None):
        """Receive rows grouped into per-expert segments padded to the aligned
        counts.  Positions the call does not write (at or past the grouped row
        total) keep the fill values: rows 0, grouped_row -2, weight NaN."""
        recv_x = np.ascontiguousarray(recv_x)
        idx = np.ascontiguousarray(recv_topk_idx, dtype=np.int64)
        w = np.ascontiguousarray(recv_topk_weights, dtype=np.float32)
        gbl = np.ascontiguousarray(recv_gbl_rank_prefix_sum, dtype=np.int32)
        aligned = np.ascontiguousarray(aligned_per_expert, dtype=np.int32)
        R, K = gbl.shape[0], idx.shape[1]
        n = idx.shape[0] if num_recv_rows is None else int(num_recv_rows)
        cap = int(aligned.sum()) if grouped_capacity is None else int(grouped_capacity)
        row_bytes = int(np.prod(recv_x.shape[1:], dtype=np.int64)) * recv_x.itemsize
        NS = 0 if recv_x_scales is None else recv_x_scales.shape[1]
        xs = None if recv_x_scales is None else np.ascontiguousarray(recv_x_scales, dtype=np.float32)
        gx = np.zeros((cap,) + recv_x.shape[1:], recv_x.dtype)
        gs = np.zeros((cap, NS), np.float32) if NS else None
        grow = np.full(cap, -2, np.int32)
        gw = np.full(cap, np.nan, np.float32)
        pos = np.zeros((n, K), np.int32)
        m = np.zeros(1, np.int32)
        st = self.lib.oracle_group_by_expert(E, R, K, row_bytes, _ptr(recv_x), _ptr(xs), NS, _ptr(idx), _ptr(w),
                                             _ptr(gbl), _ptr(aligned), n, cap, _ptr(gx), _ptr(gs), _ptr(grow),
                                             _ptr(gw), _ptr(pos), _ptr(m))
        return dict(grouped_x=gx, grouped_x_scales=gs, grouped_row=grow, grouped_weights=gw, slot_pos=pos,
                    num_grouped_rows=int(m[0]), status=st)

    def combine(self, y, recv_topk_weights, send_slot, num_recv: int, with_weights: bool = True):
        y = np.ascontiguousarray(y, dtype=np.uint16)
        recv_w = np.ascontiguousarray(recv_topk_weights, dtype=np.float32)
        send_slot = np.ascontiguousarray(send_slot, dtype=np.int32)
        T, R = send_slot.shape
        H = y.shape[1]
        K = recv_w.shape[1]
        out = np.zeros((T, H), np.uint16)
        cw = np.zeros((T, K), np.float32) if with_weights else None
        scratch = np.zeros(max(H, 1), np.float32)
        st = self.lib.oracle_combine(T, H, K, R, num_recv, _ptr(y), _ptr(recv_w), _ptr(send_slot),
                                     _ptr(out), _ptr(cw), _ptr(scratch))
        return dict(combined_x=out, combined_topk_weights=cw, status=st)

    def combine_f64(self, y, recv_topk_weights, send_slot, num_recv: int):
        y = np.ascontiguousarray(y, dtype=np.uint16)
        recv_w = np.ascontiguousarray(recv_topk_weights, dtype=np.float32)
        send_slot = np.ascontiguousarray(send_slot, dtype=np.int32)
        T, R = send_slot.shape
        H = y.shape[1]
        K = recv_w.shape[1]
        out = np.zeros((T, H), np.float64)
        st = self.lib.oracle_combine_f64(T, H, K, R, num_recv, _ptr(y), _ptr(recv_w), _ptr(send_slot),
                                         _ptr(out))
        return out, st

    def bf16_round(self, f: np.ndarray) -> np.ndarray:
        f = np.ascontiguousarray(f, dtype=np.float32)
        out = np.zeros(f.shape, np.uint16)
        self.lib.oracle_bf16_round(_ptr(f), _ptr(out), f.size)
        return out

    def e4m3_encode(self, v: np.ndarray) -> np.ndarray:
        """Nearest E4M3 pattern (ties to even) of binary32 values with |v| <= 448."""
        v = np.ascontiguousarray(v, dtype=np.float32)
        out = np.zeros(v.shape, np.uint8)
        self.lib.oracle_e4m3_encode(_ptr(v), _ptr(out), v.size)
        return out

    def e4m3_decode(self, c: np.ndarray) -> np.ndarray:
        """The value of each E4M3 pattern (binary64; NaN for S.1111.111)."""
        c = np.ascontiguousarray(c, dtype=np.uint8)
        out = np.zeros(c.shape, np.float64)
        self.lib.oracle_e4m3_decode(_ptr(c), _ptr(out), c.size)
        return out

    def quantize_e4m3(self, x: np.ndarray, num_scales: int):
        """bf16 rows [rows][H] (uint16 patterns) -> (codes uint8 [rows][H], scales f32 [rows][num_scales])."""
        x = np.ascontiguousarray(x, dtype=np.uint16)
        rows, H = x.shape
        codes = np.zeros((rows, H), np.uint8)
        scales = np.zeros((rows, num_scales), np.float32)
        rc = self.lib.oracle_quantize_e4m3(rows, H, num_scales, _ptr(x), _ptr(codes), _ptr(scales))
        if rc != 0:
            raise ValueError(f"num_scales {num_scales} does not divide hidden {H}")
        return codes, scales

    def dequantize_e4m3(self, codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
        """E4M3 codes [rows][H] and scales [rows][S] -> bf16 patterns [rows][H]."""
        codes = np.ascontiguousarray(codes, dtype=np.uint8)
        scales = np.ascontiguousarray(scales, dtype=np.float32)
        rows, H = codes.shape
        out = np.zeros((rows, H), np.uint16)
        rc = self.lib.oracle_dequantize_e4m3(rows, H, scales.shape[1], _ptr(codes), _ptr(scales), _ptr(out))
        if rc != 0:
            raise ValueError(f"num_scales {scales.shape[1]} does not divide hidden {H}")
        return out

    def full(self, x, topk_idx, topk_weights, E: int, R: int, C: int, expert_alignment: int = 1,
             my_rank: int = 0, y=None):
        """All four stages in order; combine reads ``y`` (identity experts when None)."""
        lay = self.layout(topk_idx, E, R)
        note = self.notify(lay["is_token_in_rank"], lay["num_tokens_per_rank"],
                           lay["num_tokens_per_rdma_rank"], lay["num_tokens_per_expert"], C, expert_alignment)
        dis = self.dispatch(x, topk_idx, topk_weights, lay["is_token_in_rank"],
                            note["gbl_channel_prefix_matrix"], note["recv_gbl_rank_prefix_sum"], E, my_rank)
        yy = dis["recv_x"] if y is None else y
        com = self.combine(yy, dis["recv_topk_weights"], dis["send_slot"], note["num_recv_tokens"])
        return lay, note, dis, com


def default() -> Oracle:
    return Oracle()
