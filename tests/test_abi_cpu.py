"""The C ABI on a host without a GPU: libgdn.so loads, exports every function
include/gdn.h declares, and rejects malformed arguments before touching the
device.  Device pointers here are fake; every call below carries a planted
error that the host-side checks catch, so no call ever reaches a launch."""
import ctypes

import numpy as np
import pytest

from linear_attention_causal_amd import _abi

lib = _abi.load()
V = ctypes.c_void_p
DEV = V(0x100000)       # fake, 16-byte aligned device address (never dereferenced)
DEV_ODD = V(0x100008)   # 8-byte aligned only


def geom(Hk=8, Hv=16, d=128, K=4, act=_abi.GDN_BF16, dv=None):
    return _abi.gdn_geometry(Hk, Hv, d, d if dv is None else dv, K, act, 1e-6, 1e-6, 0.0)


def weights():
    return _abi.gdn_layer_weights(DEV, DEV, DEV, DEV)


def pool(P=64):
    return _abi.gdn_state_pool(DEV, DEV, P)


def host_i32(vals):
    a = np.ascontiguousarray(np.asarray(vals, np.int32))
    return a, a.ctypes.data_as(V)


def test_exports_every_declared_function():
    names = _abi.header_functions()
    assert len(names) == 14
    for n in names:
        assert hasattr(lib, n), n
    assert set(_abi.PROTOTYPES) == set(names)
    assert lib.gdn_abi_version() == 2


def test_status_strings():
    for code in range(0, -11, -1):
        assert lib.gdn_status_str(code).decode() != "unknown status"


def test_slot_and_scratch_sizes():
    r, c = ctypes.c_size_t(), ctypes.c_size_t()
    g = geom()
    assert lib.gdn_slot_bytes(ctypes.byref(g), ctypes.byref(r), ctypes.byref(c)) == 0
    assert r.value == 16 * 128 * 128 * 4
    assert c.value == 4 * (2 * 8 * 128 + 16 * 128) * 2
    gf = geom(2, 4, 32, act=_abi.GDN_F32)
    assert lib.gdn_slot_bytes(ctypes.byref(gf), ctypes.byref(r), ctypes.byref(c)) == 0
    assert (r.value, c.value) == (4 * 32 * 32 * 4, 4 * 256 * 4)
    n1, n2 = ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.gdn_prefill_scratch_bytes(ctypes.byref(g), 64, 1, ctypes.byref(n1)) == 0
    assert lib.gdn_prefill_scratch_bytes(ctypes.byref(g), 4096, 1, ctypes.byref(n2)) == 0
    assert 0 < n1.value < n2.value
    assert lib.gdn_prefill_scratch_bytes(ctypes.byref(g), -1, 1, ctypes.byref(n1)) == _abi.GDN_E_SHAPE


@pytest.mark.parametrize("g,code", [
    (geom(Hk=3, Hv=16), _abi.GDN_E_HEADS),
    (geom(Hk=0), _abi.GDN_E_SHAPE),
    (geom(d=48), _abi.GDN_E_UNSUPPORTED),
    (geom(d=128, dv=64), _abi.GDN_E_UNSUPPORTED),
    (geom(K=5), _abi.GDN_E_UNSUPPORTED),
    (geom(K=1), _abi.GDN_E_UNSUPPORTED),
    (geom(act=7), _abi.GDN_E_UNSUPPORTED),
])
def test_geometry_rejected(g, code):
    r, c = ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.gdn_slot_bytes(ctypes.byref(g), ctypes.byref(r), ctypes.byref(c)) == code
    w, p = weights(), pool()
    rc = lib.gdn_decode_batch(ctypes.byref(g), ctypes.byref(w), ctypes.byref(p), DEV, None, 4,
                              DEV, DEV, DEV, DEV, DEV, None, None)
    assert rc == code
    assert lib.gdn_last_error().decode() != ""


def test_null_geometry():
    r, c = ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.gdn_slot_bytes(None, ctypes.byref(r), ctypes.byref(c)) == _abi.GDN_E_NULL


def _conv(B=4, slots_host=None, x=DEV, out=DEV, p=None, w=None):
    g = geom()
    w = w or weights()
    p = p or pool()
    return lib.gdn_conv_update(ctypes.byref(g), ctypes.byref(w), ctypes.byref(p), DEV,
                               slots_host, B, x, out, None)


def test_conv_update_checks():
    assert _conv(B=0) == 0                                   # no-op, nothing launched
    assert _conv(B=-1) == _abi.GDN_E_SHAPE
    assert _conv(x=None) == _abi.GDN_E_NULL
    assert _conv(out=DEV_ODD) == _abi.GDN_E_ALIGN
    _, h = host_i32([0, 1, 64, 2])
    assert _conv(slots_host=h) == _abi.GDN_E_SLOT            # out of range
    _, h = host_i32([0, 5, -1, 5])
    assert _conv(slots_host=h) == _abi.GDN_E_SLOT            # duplicate
    assert _conv(p=_abi.gdn_state_pool(DEV, None, 64)) == _abi.GDN_E_NULL
    assert _conv(p=_abi.gdn_state_pool(DEV, DEV, 0)) == _abi.GDN_E_SHAPE
    assert _conv(w=_abi.gdn_layer_weights(DEV, None, DEV, DEV)) == _abi.GDN_E_NULL


def _decode(B=4, slots_host=None, z=DEV, o_raw=None):
    g, w, p = geom(), weights(), pool()
    return lib.gdn_decode_batch(ctypes.byref(g), ctypes.byref(w), ctypes.byref(p), DEV,
                                slots_host, B, DEV, z, DEV, DEV, DEV, o_raw, None)


def test_decode_batch_checks():
    assert _decode(B=0) == 0
    assert _decode(B=-2) == _abi.GDN_E_SHAPE
    assert _decode(z=None) == _abi.GDN_E_NULL
    assert _decode(o_raw=DEV_ODD) == _abi.GDN_E_ALIGN
    _, h = host_i32([3, -1, 63, 3])
    assert _decode(slots_host=h) == _abi.GDN_E_SLOT


def _ws_bytes(g, B):
    n = ctypes.c_size_t()
    assert lib.gdn_decode_workspace_bytes(ctypes.byref(g), B, ctypes.byref(n)) == 0
    return n.value


def test_decode_workspace_sizes():
    """The workspace scales with the rows, not the pool, and a workspace sized
    for B rows serves every smaller call (the size never decreases with B)."""
    for g in (geom(), geom(Hk=16, Hv=32), geom(Hk=2, Hv=4, d=32), geom(Hk=4, Hv=16, d=64)):
        sizes = [_ws_bytes(g, B) for B in range(0, 300)]
        assert all(a <= b for a, b in zip(sizes, sizes[1:]))
        assert all(x % 256 == 0 for x in sizes)
    # q/k counters alone past the split rows: B * Hk * (2 d / 64) words
    g = geom(Hk=16, Hv=32)
    big = _ws_bytes(g, 4096) - _ws_bytes(g, 2048)
    assert big == 2048 * 16 * 4 * 4
    n = ctypes.c_size_t()
    assert lib.gdn_decode_workspace_bytes(ctypes.byref(g), -1, ctypes.byref(n)) == \
        _abi.GDN_E_SHAPE
    assert lib.gdn_decode_workspace_bytes(ctypes.byref(g), 4, None) == _abi.GDN_E_NULL


def test_decode_step_checks():
    """gdn_decode_step: any Hv/Hk and any pool size; the workspace is checked
    (missing, too small, misaligned) before anything is enqueued.  Every call
    below carries a planted error, so none reaches a launch."""
    def step(g, P=64, B=4, ws=V(0x400000), nbytes=1 << 30, z=DEV):
        w, p = weights(), pool(P)
        return lib.gdn_decode_step(ctypes.byref(g), ctypes.byref(w), ctypes.byref(p), DEV, None,
                                   B, DEV, z, DEV, DEV, DEV, None, ws, nbytes, None)
    g = geom()
    assert step(g, B=0, ws=None, nbytes=0) == 0                  # empty: no-op
    assert step(g, B=-1) == _abi.GDN_E_SHAPE
    assert step(g, ws=None) == _abi.GDN_E_SCRATCH
    assert step(g, nbytes=_ws_bytes(g, 4) - 1) == _abi.GDN_E_SCRATCH
    assert step(g, ws=V(0x400010)) == _abi.GDN_E_ALIGN
    assert step(g, z=None) == _abi.GDN_E_NULL
    assert step(geom(Hk=2, Hv=6, d=32), P=1 << 20, ws=None) == _abi.GDN_E_SCRATCH
    assert b"workspace" in lib.gdn_last_error()


def test_decode_step_noalloc_checks():
    """gdn_decode_step_noalloc validates like gdn_decode_step and rejects row
    counts whose workspace exceeds the 1 MiB the library holds per GPU, all
    before touching the device (every call below returns before a launch)."""
    def step(g, B=4, z=DEV):
        w, p = weights(), pool(64)
        return lib.gdn_decode_step_noalloc(ctypes.byref(g), ctypes.byref(w), ctypes.byref(p),
                                           DEV, None, B, DEV, z, DEV, DEV, DEV, None, None)
    g = geom(Hk=16, Hv=32)
    assert step(g, B=0) == 0
    assert step(g, B=-1) == _abi.GDN_E_SHAPE
    assert step(g, z=None) == _abi.GDN_E_NULL
    assert _ws_bytes(g, 4096) == 1 << 20 and _ws_bytes(g, 4097) > 1 << 20
    assert step(g, B=4097) == _abi.GDN_E_SCRATCH
    assert b"1048576" in lib.gdn_last_error()


def _prefill(cu, slots_host=None, scratch=DEV, nbytes=1 << 40, N=None):
    g, w, p = geom(), weights(), pool()
    cu_a, cu_p = host_i32(cu)
    N = len(cu) - 1 if N is None else N
    return lib.gdn_prefill_chunked(ctypes.byref(g), ctypes.byref(w), ctypes.byref(p), cu_p,
                                   DEV, DEV, slots_host, None, N, DEV, DEV, DEV, DEV, DEV,
                                   None, scratch, nbytes, None)


def test_prefill_checks():
    assert _prefill([0], N=0) == 0
    assert _prefill([1, 10]) == _abi.GDN_E_SEQLENS
    assert _prefill([0, 10, 5]) == _abi.GDN_E_SEQLENS
    assert _prefill([0, 100], nbytes=1024) == _abi.GDN_E_SCRATCH
    assert _prefill([0, 100], scratch=None) == _abi.GDN_E_SCRATCH
    assert _prefill([0, 100], scratch=V(0x100010)) == _abi.GDN_E_ALIGN
    _, h = host_i32([1, 1])
    assert _prefill([0, 5, 9], slots_host=h) == _abi.GDN_E_SLOT
    assert _prefill([0, 5], N=70000) == _abi.GDN_E_SHAPE


def _compact(src, dst, pools=None):
    g = geom()
    pools = pools or [pool(8), pool(8)]
    arr = (_abi.gdn_state_pool * len(pools))(*pools)
    s, sp = host_i32(src)
    d, dp = host_i32(dst)
    return lib.gdn_state_compact(ctypes.byref(g), arr, len(pools), sp, dp, DEV, DEV, len(s),
                                 None)


def test_compact_checks():
    assert _compact([], []) == 0
    assert _compact([5, 6], [1, 6]) == _abi.GDN_E_OVERLAP       # 6 is both
    assert _compact([5, 6], [1, 1]) == _abi.GDN_E_SLOT          # dst twice
    assert _compact([5, 8], [1, 2]) == _abi.GDN_E_SLOT          # out of range
    assert _compact([5, 6], [1, 5]) == _abi.GDN_E_OVERLAP
    assert _compact([5], [1], pools=[pool(8), pool(9)]) == _abi.GDN_E_SHAPE


def _lin(M=16, K=64, ldx=64, outs=None, count=None, x=DEV):
    if outs is None:
        outs = [(V(0x200000), V(0x300000), 32, 32)]
    arr = (_abi.gdn_linear_out * max(len(outs), 1))(
        *[_abi.gdn_linear_out(w, y, n, ld) for (w, y, n, ld) in outs])
    return lib.gdn_linear(x, M, K, ldx, arr, len(outs) if count is None else count, None)


def test_linear_validation():
    """Every check of gdn_linear returns before anything is enqueued."""
    assert _lin(M=0, x=None) == _abi.GDN_OK                      # empty: no-op
    assert _lin(M=-1) == _abi.GDN_E_SHAPE
    assert _lin(K=60, ldx=64) == _abi.GDN_E_SHAPE                # K % 8
    assert _lin(K=64, ldx=32) == _abi.GDN_E_SHAPE                # ldx < K
    assert _lin(K=64, ldx=68) == _abi.GDN_E_SHAPE                # ldx % 8
    assert _lin(count=0) == _abi.GDN_E_SHAPE
    assert _lin(outs=[(V(0x200000), V(0x300000), 32, 32)] * 5) == _abi.GDN_E_SHAPE
    assert _lin(x=None) == _abi.GDN_E_NULL
    assert _lin(x=DEV_ODD) == _abi.GDN_E_ALIGN
    assert _lin(outs=[(None, V(0x300000), 32, 32)]) == _abi.GDN_E_NULL
    assert _lin(outs=[(V(0x200008), V(0x300000), 32, 32)]) == _abi.GDN_E_ALIGN
    assert _lin(outs=[(V(0x200000), V(0x300001), 32, 32)]) == _abi.GDN_E_ALIGN
    assert _lin(outs=[(V(0x200000), V(0x300000), 32, 16)]) == _abi.GDN_E_SHAPE   # ldy < N
    assert _lin(outs=[(V(0x200000), V(0x300000), 0, 32)]) == _abi.GDN_E_SHAPE
    # x spans [DEV, DEV + 2 (15 * 64 + 64)) = 2048 bytes: an output starting at
    # its last element overlaps
    assert _lin(outs=[(V(0x200000), V(0x100000 + 2046), 32, 32)]) == _abi.GDN_E_OVERLAP
    # an output over a weight, and two outputs over each other
    assert _lin(outs=[(V(0x200000), V(0x200000 + 64), 32, 32)]) == _abi.GDN_E_OVERLAP
    assert _lin(outs=[(V(0x200000), V(0x300000), 32, 32),
                      (V(0x400000), V(0x300000 + 1000), 32, 32)]) == _abi.GDN_E_OVERLAP
    assert b"overlap" in lib.gdn_last_error()


def test_check_slots_validation():
    """gdn_check_slots rejects bad arguments before any launch."""
    assert lib.gdn_check_slots(DEV, -1, 64, DEV, None) == _abi.GDN_E_SHAPE
    assert lib.gdn_check_slots(DEV, (1 << 20) + 1, 64, DEV, None) == _abi.GDN_E_SHAPE
    assert lib.gdn_check_slots(DEV, 4, 0, DEV, None) == _abi.GDN_E_SHAPE
    assert lib.gdn_check_slots(None, 4, 64, DEV, None) == _abi.GDN_E_NULL
    assert lib.gdn_check_slots(DEV, 4, 64, None, None) == _abi.GDN_E_NULL
    assert lib.gdn_check_slots(DEV, 4, 64, V(0x100002), None) == _abi.GDN_E_ALIGN
