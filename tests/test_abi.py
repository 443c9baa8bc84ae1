"""The C ABI without a GPU: libep.so loads, exports every entry point that
include/ep.h declares, and rejects malformed arguments on the host before
anything is launched (so these calls never touch a device)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ep.h")


@pytest.fixture(scope="module")
def ep():
    from combine_ep_get_02_amd import ep as ep_mod

    if not os.path.exists(ep_mod.LIBRARY):
        import __graft_entry__

        __graft_entry__.build()
    ep_mod.load()
    return ep_mod


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ep_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(["ep_get_layout", "ep_get_layout_noalloc", "ep_notify", "ep_layout_notify",
                                          "ep_dispatch",
                                          "ep_dispatch_fp8", "ep_quantize_fp8", "ep_dequantize_fp8",
                                          "ep_dispatch_to_fp8", "ep_dispatch_cached_to_fp8",
                                          "ep_dispatch_cached", "ep_group_by_expert", "ep_dispatch_grouped",
                                          "ep_combine", "ep_workspace_bytes", "ep_status_string"])


def test_library_exports_every_declared_symbol(ep):
    out = subprocess.run(["nm", "-D", "--defined-only", ep.LIBRARY], capture_output=True, text=True, check=True)
    exported = set(re.findall(r"\bT (ep_\w+)", out.stdout))
    missing = [f for f in declared_functions() if f not in exported]
    assert not missing, missing
    assert set(ep.EXPORTED) == set(declared_functions())


def test_status_strings(ep):
    for code in range(4):
        assert ep.ep_status_string(code).startswith(("EP_OK", "EP_ERR"))


def test_workspace_bytes(ep):
    s = ep.make_shape(4096, 7168, 8, 256, 64, 24)
    n = ep.ep_workspace_bytes(s)
    # tickets 256 + running counts (64+8+256) + masks (8 B/token) + 64 x 64 chunk offsets
    # + 16 x 64 and 16 x 8 group offsets (four chunks a group) + 24 x 64 + 24 x 8 channel-end
    # values, each 256-aligned
    assert n == 256 + 1536 + 32768 + 16384 + 4096 + 512 + 6144 + 768
    assert ep.ep_workspace_bytes(ep.make_shape(4096, 7168, 8, 255, 64, 24)) == 0  # E % R != 0


BAD_SHAPES = {
    "negative tokens": dict(num_tokens=-1),
    "hidden not /8": dict(hidden=12),
    "hidden zero": dict(hidden=0),
    "topk zero": dict(num_topk=0),
    "experts not /R": dict(num_experts=100),
    "ranks 12": dict(num_ranks=12, num_experts=96),
    "channels zero": dict(num_channels=0),
    "my_rank out": dict(my_rank=64),
    "alignment zero": dict(expert_alignment=0),
}
UNSUPPORTED = {"ranks 72": dict(num_ranks=72, num_experts=288), "topk 33": dict(num_topk=33),
               "channels 5000": dict(num_channels=5000)}


def _shape(ep, **kw):
    base = dict(num_tokens=4096, hidden=7168, num_topk=8, num_experts=256, num_ranks=64, num_channels=24,
                my_rank=0, expert_alignment=1)
    base.update(kw)
    return ep.make_shape(**base)


def _call_all(ep, s):
    lib = ep.load()
    p = ctypes.c_void_p(256)  # never dereferenced: every call must fail its host checks first
    codes = [
        lib.ep_get_layout(ctypes.byref(s), p, p, p, p, p, p, 1 << 30, None, None),
        lib.ep_notify(ctypes.byref(s), p, p, p, p, p, p, p, p, p, p, None, p, 1 << 30, None, None),
        lib.ep_layout_notify(ctypes.byref(s), p, p, p, p, p, p, p, p, p, p, p, None, p, 1 << 30, None, None),
        lib.ep_dispatch(ctypes.byref(s), p, p, p, p, p, p, p, 1 << 30, 10, p, p, None, p, p, 0, None, None),
        lib.ep_combine(ctypes.byref(s), p, p, p, 10, p, None, None, None),
        lib.ep_dispatch_fp8(ctypes.byref(s), p, p, 4, p, p, p, p, p, p, 1 << 30, 10, p, p, p, None, p, p, 0,
                            None, None),
        lib.ep_dispatch_cached(ctypes.byref(s), p, 2, None, 0, p, 10, p, None, 0, None, None),
        lib.ep_group_by_expert(ctypes.byref(s), p, 2, None, 0, p, p, p, p, 10, 10, p, None, p, p, p, p, None, None),
    ]
    return codes


@pytest.mark.parametrize("name", sorted(BAD_SHAPES))
def test_malformed_shapes_rejected(ep, name):
    assert _call_all(ep, _shape(ep, **BAD_SHAPES[name])) == [ep.EP_ERR_INVALID_ARG] * 8


@pytest.mark.parametrize("name", sorted(UNSUPPORTED))
def test_unsupported_shapes_rejected(ep, name):
    assert _call_all(ep, _shape(ep, **UNSUPPORTED[name])) == [ep.EP_ERR_UNSUPPORTED] * 8


def test_null_and_misaligned_pointers_rejected(ep):
    lib = ep.load()
    s = _shape(ep)
    p = ctypes.c_void_p(256)
    odd = ctypes.c_void_p(264)
    assert lib.ep_get_layout(ctypes.byref(s), None, p, p, p, p, p, 1 << 30, None, None) == ep.EP_ERR_INVALID_ARG
    assert lib.ep_get_layout(ctypes.byref(s), p, p, p, p, p, p, 16, None, None) == ep.EP_ERR_INVALID_ARG
    assert lib.ep_notify(ctypes.byref(s), p, p, p, p, p, p, p, p, p, p, None, None, 1 << 30, None,
                         None) == ep.EP_ERR_INVALID_ARG  # no workspace
    assert lib.ep_notify(ctypes.byref(s), p, p, p, p, p, p, p, p, p, p, None, p, 16, None,
                         None) == ep.EP_ERR_INVALID_ARG  # workspace too small
    assert lib.ep_dispatch(ctypes.byref(s), odd, p, p, p, p, p, p, 1 << 30, 10, p, p, None, p, p, 0, None,
                           None) == ep.EP_ERR_INVALID_ARG  # x not 16-byte aligned
    assert lib.ep_dispatch(ctypes.byref(s), p, p, p, p, p, p, p, 1 << 30, -1, p, p, None, p, p, 0, None,
                           None) == ep.EP_ERR_INVALID_ARG  # negative capacity
    assert lib.ep_dispatch(ctypes.byref(s), p, p, p, None, p, p, p, 1 << 30, 10, p, p, None, p, p, 0, None,
                           None) == ep.EP_ERR_INVALID_ARG  # no is_token_in_rank
    assert lib.ep_dispatch(ctypes.byref(s), p, p, p, p, None, p, p, 1 << 30, 10, p, p, None, p, p, 0, None,
                           None) == ep.EP_ERR_INVALID_ARG  # no channel prefix matrix
    assert lib.ep_dispatch(ctypes.byref(s), p, p, p, p, p, None, p, 1 << 30, 10, p, p, None, p, p, 0, None,
                           None) == ep.EP_ERR_INVALID_ARG  # no receive prefix sums
    assert lib.ep_dispatch(ctypes.byref(s), p, p, p, p, p, p, p, 16, 10, p, p, None, p, p, 0, None,
                           None) == ep.EP_ERR_INVALID_ARG  # workspace given but too small
    assert lib.ep_combine(ctypes.byref(s), p, p, p, 10, odd, None, None, None) == ep.EP_ERR_INVALID_ARG
    assert lib.ep_combine(ctypes.byref(s), p, p, None, 10, p, None, None, None) == ep.EP_ERR_INVALID_ARG
    assert lib.ep_get_layout(None, p, p, p, p, p, p, 1 << 30, None, None) == ep.EP_ERR_INVALID_ARG


def test_fp8_and_cached_argument_checks(ep):
    lib = ep.load()
    p = ctypes.c_void_p(256)
    s = _shape(ep)
    # fp8 rows must be a whole number of 16-byte units
    s12 = _shape(ep, hidden=7160)
    assert lib.ep_dispatch_fp8(ctypes.byref(s12), p, p, 4, p, p, p, p, p, p, 1 << 30, 10, p, p, p, None, p, p, 0,
                               None, None) == ep.EP_ERR_INVALID_ARG
    assert lib.ep_dispatch_fp8(ctypes.byref(s), p, None, 4, p, p, p, p, p, p, 1 << 30, 10, p, p, p, None, p, p, 0,
                               None, None) == ep.EP_ERR_INVALID_ARG  # scales missing
    assert lib.ep_dispatch_fp8(ctypes.byref(s), p, p, 2000, p, p, p, p, p, p, 1 << 30, 10, p, p, p, None, p, p, 0,
                               None, None) == ep.EP_ERR_UNSUPPORTED
    assert lib.ep_dispatch_cached(ctypes.byref(s), p, 3, None, 0, p, 10, p, None, 0, None, None) == ep.EP_ERR_INVALID_ARG
    assert lib.ep_dispatch_cached(ctypes.byref(s), p, 2, None, 0, None, 10, p, None, 0, None, None) == ep.EP_ERR_INVALID_ARG
    assert lib.ep_dispatch_cached(ctypes.byref(s12), p, 1, None, 0, p, 10, p, None, 0, None, None) == ep.EP_ERR_INVALID_ARG


def test_quantize_argument_checks(ep):
    lib = ep.load()
    p = ctypes.c_void_p(256)
    for fn in (lambda *a: lib.ep_quantize_fp8(p, a[0], a[1], a[2], p, p, None),
               lambda *a: lib.ep_dequantize_fp8(p, p, a[0], a[1], a[2], p, None)):
        assert fn(-1, 7168, 56) == ep.EP_ERR_INVALID_ARG      # negative row count
        assert fn(4, 7160, 56) == ep.EP_ERR_INVALID_ARG       # hidden not a multiple of 16
        assert fn(4, 0, 1) == ep.EP_ERR_INVALID_ARG
        assert fn(4, 7168, 0) == ep.EP_ERR_INVALID_ARG
        assert fn(4, 7168, 3) == ep.EP_ERR_INVALID_ARG        # 3 does not divide 7168
        assert fn(4, 7168, 64) == ep.EP_ERR_UNSUPPORTED       # groups of 112 channels
        assert fn(4, 4096, 2) == ep.EP_ERR_UNSUPPORTED        # groups of 2048 channels
        assert fn(4, 96, 12) == ep.EP_ERR_UNSUPPORTED         # groups of 8 channels
        assert fn(0, 7168, 56) == ep.EP_OK                    # nothing to do, nothing enqueued
    s = _shape(ep)
    d = lambda sh, S, **kw: lib.ep_dispatch_to_fp8(ctypes.byref(sh), kw.get("x", p), S, p, p, p, p, p, None, 0,  # noqa: E731
                                                   kw.get("cap", 10), p, kw.get("rs", p), p, p, p, p, None, None)
    assert d(s, 3) == ep.EP_ERR_INVALID_ARG                    # 3 does not divide hidden
    assert d(s, 64) == ep.EP_ERR_UNSUPPORTED                   # groups of 112 channels
    assert d(_shape(ep, hidden=7160), 1) == ep.EP_ERR_INVALID_ARG
    assert d(s, 56, rs=None) == ep.EP_ERR_INVALID_ARG          # scales out missing
    assert d(s, 56, x=ctypes.c_void_p(264)) == ep.EP_ERR_INVALID_ARG  # x not 16-byte aligned
    assert d(s, 56, x=None) == ep.EP_ERR_INVALID_ARG
    assert d(_shape(ep, hidden=0), 1) == ep.EP_ERR_INVALID_ARG  # the shape is checked first
    assert lib.ep_dispatch_to_fp8(None, p, 56, p, p, p, p, p, None, 0, 10, p, p, p, p, p, p, None, None) == \
        ep.EP_ERR_INVALID_ARG
    assert d(_shape(ep, num_tokens=0), 56) == ep.EP_OK            # no tokens: nothing to do, nothing enqueued
    cq = lambda sh, S, **kw: lib.ep_dispatch_cached_to_fp8(ctypes.byref(sh), kw.get("x", p), S,  # noqa: E731
                                                           kw.get("slot", p), kw.get("cap", 10), kw.get("rx", p),
                                                           kw.get("rs", p), None, None)
    assert cq(s, 3) == ep.EP_ERR_INVALID_ARG
    assert cq(s, 64) == ep.EP_ERR_UNSUPPORTED
    assert cq(_shape(ep, hidden=7160), 1) == ep.EP_ERR_INVALID_ARG
    assert cq(s, 56, cap=-1) == ep.EP_ERR_INVALID_ARG
    assert cq(s, 56, slot=None) == ep.EP_ERR_INVALID_ARG
    assert cq(s, 56, rs=None) == ep.EP_ERR_INVALID_ARG
    assert cq(s, 56, rx=ctypes.c_void_p(264)) == ep.EP_ERR_INVALID_ARG
    assert cq(_shape(ep, num_tokens=0), 56) == ep.EP_OK
    q = ctypes.c_void_p(264)  # 8-byte aligned only
    assert lib.ep_quantize_fp8(q, 4, 7168, 56, p, p, None) == ep.EP_ERR_INVALID_ARG
    assert lib.ep_quantize_fp8(p, 4, 7168, 56, q, p, None) == ep.EP_ERR_INVALID_ARG
    assert lib.ep_quantize_fp8(p, 4, 7168, 56, p, ctypes.c_void_p(258), None) == ep.EP_ERR_INVALID_ARG
    assert lib.ep_quantize_fp8(None, 4, 7168, 56, p, p, None) == ep.EP_ERR_INVALID_ARG
    assert lib.ep_dequantize_fp8(p, None, 4, 7168, 56, p, None) == ep.EP_ERR_INVALID_ARG
    assert lib.ep_dequantize_fp8(p, p, 4, 7168, 56, q, None) == ep.EP_ERR_INVALID_ARG


def test_group_by_expert_argument_checks(ep):
    lib = ep.load()
    p = ctypes.c_void_p(256)
    odd = ctypes.c_void_p(264)
    s = _shape(ep)

    def group(shape=s, recv_x=p, elem=2, scales=None, ns=0, idx=p, w=p, gbl=p, aligned=p, rows=10, cap=10,
              gx=p, gscales=None, grow=p, gw=p, pos=p, m=p):
        return lib.ep_group_by_expert(ctypes.byref(shape), recv_x, elem, scales, ns, idx, w, gbl, aligned, rows, cap,
                                      gx, gscales, grow, gw, pos, m, None, None)

    assert group(elem=3) == ep.EP_ERR_INVALID_ARG
    assert group(shape=_shape(ep, hidden=7160), elem=1) == ep.EP_ERR_INVALID_ARG  # not whole 16-byte units
    assert group(rows=-1) == ep.EP_ERR_INVALID_ARG
    assert group(cap=-1) == ep.EP_ERR_INVALID_ARG
    assert group(m=None) == ep.EP_ERR_INVALID_ARG  # num_grouped_rows is required
    assert group(gbl=None) == ep.EP_ERR_INVALID_ARG
    assert group(aligned=None) == ep.EP_ERR_INVALID_ARG
    assert group(idx=None) == ep.EP_ERR_INVALID_ARG
    assert group(grow=None) == ep.EP_ERR_INVALID_ARG
    assert group(w=None) == ep.EP_ERR_INVALID_ARG  # grouped weights need the receive weights
    assert group(ns=4) == ep.EP_ERR_INVALID_ARG  # scales missing
    assert group(gx=odd) == ep.EP_ERR_INVALID_ARG
    assert group(recv_x=odd) == ep.EP_ERR_INVALID_ARG
    assert group(ns=2000, scales=p, gscales=p) == ep.EP_ERR_UNSUPPORTED
    assert group(shape=_shape(ep, num_experts=1024, num_ranks=1)) == ep.EP_ERR_UNSUPPORTED  # 1024 local experts
    assert group(rows=(1 << 31) // 8) == ep.EP_ERR_UNSUPPORTED  # rows * k reaches 2^31


def test_dispatch_grouped_argument_checks(ep):
    # every call below breaks exactly one rule, so it is refused before any launch
    lib = ep.load()
    p = ctypes.c_void_p(256)
    odd = ctypes.c_void_p(264)
    s = _shape(ep)

    def grouped(shape=s, x=p, elem=2, xs=None, ns=0, idx=p, w=p, in_rank=p, cpm=p, gbl=p, aligned=p, ws=p,
                wsb=1 << 30, cap=10, rw=p, ridx=p, src=p, slot=p, gcap=10, gx=p, gxs=None, grow=p, gw=p, pos=p, m=p):
        return lib.ep_dispatch_grouped(ctypes.byref(shape), x, elem, xs, ns, idx, w, in_rank, cpm, gbl, aligned, ws,
                                       wsb, cap, rw, ridx, src, slot, gcap, gx, gxs, grow, gw, pos, m, None, None)

    assert grouped(elem=3) == ep.EP_ERR_INVALID_ARG
    assert grouped(shape=_shape(ep, hidden=7160), elem=1) == ep.EP_ERR_INVALID_ARG  # not whole 16-byte units
    assert grouped(cap=-1) == ep.EP_ERR_INVALID_ARG
    assert grouped(gcap=-1) == ep.EP_ERR_INVALID_ARG
    assert grouped(m=None) == ep.EP_ERR_INVALID_ARG
    assert grouped(gbl=None) == ep.EP_ERR_INVALID_ARG
    assert grouped(aligned=None) == ep.EP_ERR_INVALID_ARG
    assert grouped(ridx=None) == ep.EP_ERR_INVALID_ARG  # the grouping reads the receive ids
    assert grouped(rw=None) == ep.EP_ERR_INVALID_ARG
    assert grouped(src=None) == ep.EP_ERR_INVALID_ARG
    assert grouped(pos=None) == ep.EP_ERR_INVALID_ARG  # the rows are stored through slot_pos
    assert grouped(src=ctypes.c_void_p(260)) == ep.EP_ERR_INVALID_ARG  # src_info is 8-byte aligned
    assert grouped(grow=None) == ep.EP_ERR_INVALID_ARG
    assert grouped(gx=odd) == ep.EP_ERR_INVALID_ARG
    assert grouped(x=odd) == ep.EP_ERR_INVALID_ARG
    assert grouped(x=None) == ep.EP_ERR_INVALID_ARG
    assert grouped(idx=None) == ep.EP_ERR_INVALID_ARG
    assert grouped(w=None) == ep.EP_ERR_INVALID_ARG
    assert grouped(slot=None) == ep.EP_ERR_INVALID_ARG
    assert grouped(wsb=10) == ep.EP_ERR_INVALID_ARG  # short workspace
    assert grouped(ws=None, wsb=0) == ep.EP_ERR_INVALID_ARG  # the grouped dispatch needs its workspace
    assert grouped(in_rank=None) == ep.EP_ERR_INVALID_ARG
    assert grouped(cpm=None) == ep.EP_ERR_INVALID_ARG
    assert grouped(ns=4, gxs=p) == ep.EP_ERR_INVALID_ARG  # x scales missing
    assert grouped(ns=4, xs=p) == ep.EP_ERR_INVALID_ARG  # grouped scales missing
    assert grouped(ns=2000, xs=p, gxs=p) == ep.EP_ERR_UNSUPPORTED
    assert grouped(shape=_shape(ep, num_experts=1024, num_ranks=1)) == ep.EP_ERR_UNSUPPORTED  # 1024 local experts
    assert grouped(cap=(1 << 31) // 8) == ep.EP_ERR_UNSUPPORTED  # rows * k reaches 2^31


def test_empty_dispatch_and_combine_enqueue_nothing(ep):
    # t = 0: nothing to move; the calls succeed without touching any pointer
    lib = ep.load()
    s = _shape(ep, num_tokens=0)
    assert lib.ep_dispatch(ctypes.byref(s), None, None, None, None, None, None, None, 0, 0, None, None, None, None,
                           None, 0, None, None) == ep.EP_OK
    assert lib.ep_combine(ctypes.byref(s), None, None, None, 0, None, None, None, None) == ep.EP_OK


def test_dispatch_without_workspace_limits(ep):
    # without a workspace the routing is worked out inside the call, counting at most
    # half a channel per chunk: channels of up to 4096 tokens are accepted, longer
    # ones need the workspace notify filled (refused before any launch otherwise)
    lib = ep.load()
    p = ctypes.c_void_p(256)

    def dispatch(shape, ws, wsb):
        return lib.ep_dispatch(ctypes.byref(shape), p, p, p, p, p, p, ws, wsb, 10, p, p, None, p, p, 0, None, None)

    long_channels = _shape(ep, num_tokens=100000, num_channels=24)  # 4167 tokens per channel
    assert dispatch(long_channels, None, 0) == ep.EP_ERR_UNSUPPORTED
    fp8 = lib.ep_dispatch_fp8(ctypes.byref(long_channels), p, p, 4, p, p, p, p, p, None, 0, 10, p, p, p, None, p, p, 0,
                              None, None)
    assert fp8 == ep.EP_ERR_UNSUPPORTED


def test_noalloc_layout_argument_checks(ep):
    # refused on the host before any device call: a shape beyond the static scratch,
    # malformed shapes, missing outputs
    lib = ep.load()
    p = ctypes.c_void_p(256)

    def call(shape, idx=p, rank=p, node=p, expert=p, in_rank=p):
        return lib.ep_get_layout_noalloc(ctypes.byref(shape), idx, rank, node, expert, in_rank, None, None)

    assert call(_shape(ep, num_experts=16384 * 2, num_ranks=64)) == ep.EP_ERR_UNSUPPORTED
    assert call(_shape(ep, num_ranks=12)) == ep.EP_ERR_INVALID_ARG
    assert call(_shape(ep), rank=None) == ep.EP_ERR_INVALID_ARG
    assert call(_shape(ep), in_rank=None) == ep.EP_ERR_INVALID_ARG
    assert call(_shape(ep), idx=None) == ep.EP_ERR_INVALID_ARG


def test_device_status_bits_agree_with_the_header(ep):
    # the binding's EP_DEV_* values are the header's (EP_DEV_STALE_WORKSPACE among them)
    text = open(HEADER).read()
    bits = dict((m.group(1), int(m.group(2))) for m in re.finditer(r"\b(EP_DEV_[A-Z_]+)\s*=\s*(\d+)", text))
    assert bits == {name: getattr(ep, name) for name in bits}
    assert bits["EP_DEV_STALE_WORKSPACE"] == 16 and len(set(bits.values())) == len(bits) == 5


def test_dispatch_form_must_be_known(ep):
    # form is one of EP_FORM_AUTO, EP_FORM_PUSH, EP_FORM_PULL; anything else is refused on the host
    lib = ep.load()
    p = ctypes.c_void_p(256)
    s = _shape(ep)
    assert (ep.EP_FORM_AUTO, ep.EP_FORM_PUSH, ep.EP_FORM_PULL) == (0, 1, 2)
    for form in (-1, 3, 7):
        assert lib.ep_dispatch(ctypes.byref(s), p, p, p, p, p, p, p, 1 << 30, 10, p, p, None, p, p, form, None,
                               None) == ep.EP_ERR_INVALID_ARG
        assert lib.ep_dispatch_fp8(ctypes.byref(s), p, p, 4, p, p, p, p, p, p, 1 << 30, 10, p, p, p, None, p, p, form,
                                   None, None) == ep.EP_ERR_INVALID_ARG
        assert lib.ep_dispatch_cached(ctypes.byref(s), p, 2, None, 0, p, 10, p, None, form, None,
                                      None) == ep.EP_ERR_INVALID_ARG


def test_cached_dispatch_has_no_pull_form(ep):
    # cached mode copies rows with the push form only: EP_FORM_PULL is refused on the host
    lib = ep.load()
    p = ctypes.c_void_p(256)
    s = _shape(ep)
    assert lib.ep_dispatch_cached(ctypes.byref(s), p, 2, None, 0, p, 10, p, None, ep.EP_FORM_PULL, None,
                                  None) == ep.EP_ERR_UNSUPPORTED


def test_layout_notify_argument_checks(ep):
    lib = ep.load()
    p = ctypes.c_void_p(256)
    s = _shape(ep)

    def call(idx=p, rank=p, gbl=p, n=p, ws=p, wsb=1 << 30, in_rank=p):
        return lib.ep_layout_notify(ctypes.byref(s), idx, rank, p, p, in_rank, gbl, p, p, p, p, n, None, ws, wsb, None,
                                    None)

    assert call(idx=None) == ep.EP_ERR_INVALID_ARG
    assert call(in_rank=None) == ep.EP_ERR_INVALID_ARG
    assert call(rank=None) == ep.EP_ERR_INVALID_ARG
    assert call(gbl=None) == ep.EP_ERR_INVALID_ARG
    assert call(n=None) == ep.EP_ERR_INVALID_ARG
    assert call(ws=None) == ep.EP_ERR_INVALID_ARG
    assert call(wsb=16) == ep.EP_ERR_INVALID_ARG
