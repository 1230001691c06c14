"""Double-precision CPU oracle of the Gated DeltaNet layer.

TEST INFRASTRUCTURE ONLY: the test-suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The GPU package never imports this
module and this module never imports the GPU package.

`gdn_oracle.c` holds the arithmetic (token-by-token gated delta rule in f64,
plus the blocked rewriting used only to check the blocked algebra);
`bruteforce.py` holds an independent numpy transition-matrix form for tiny
shapes.  This file only marshals numpy arrays to the C library.

Every function takes inputs exactly as the GPU receives them (already rounded
to their storage type) and computes in double with no intermediate rounding.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

from .build import LIB, build_oracle

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build_oracle()
        lib = ctypes.CDLL(LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        ip = ctypes.POINTER(ctypes.c_int)
        up = ctypes.c_void_p
        gp = ctypes.POINTER(_Geom)
        wp = ctypes.POINTER(_Weights)
        lib.ogdn_sequences.argtypes = [gp, wp, ctypes.c_int, ip, dp, dp, dp, dp,
                                       dp, dp, dp, dp, up, ctypes.c_int, ctypes.c_int]
        lib.ogdn_sequences.restype = ctypes.c_int
        lib.ogdn_pool_run.argtypes = [gp, wp, dp, dp, ctypes.c_int, ctypes.c_int,
                                      ip, ip, up, dp, dp, dp, dp, dp, dp, ctypes.c_int]
        lib.ogdn_pool_run.restype = ctypes.c_int
        lib.ogdn_compact.argtypes = [gp, dp, dp, ctypes.c_int, ip, ip, ctypes.c_int]
        lib.ogdn_compact.restype = ctypes.c_int
        lib.ogdn_silu.argtypes = [ctypes.c_double]
        lib.ogdn_silu.restype = ctypes.c_double
        lib.ogdn_softplus.argtypes = [ctypes.c_double]
        lib.ogdn_softplus.restype = ctypes.c_double
        lib.ogdn_gates.argtypes = [ctypes.c_double] * 4 + [dp, dp]
        lib.ogdn_l2norm.argtypes = [dp, ctypes.c_int, ctypes.c_double, ctypes.c_double, dp]
        lib.ogdn_gdr_step.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                      ctypes.c_double, dp, dp, dp, dp, dp]
        lib.ogdn_gated_rmsnorm.argtypes = [ctypes.c_int, dp, dp, dp, ctypes.c_double, dp]
        lib.ogdn_conv_channel.argtypes = [ctypes.c_int, ctypes.c_int, dp, dp, dp,
                                          ctypes.c_int, ctypes.c_int, dp, dp, ctypes.c_int]
        _lib = lib
    return _lib


class _Geom(ctypes.Structure):
    _fields_ = [("num_k_heads", ctypes.c_int), ("num_v_heads", ctypes.c_int),
                ("head_k_dim", ctypes.c_int), ("head_v_dim", ctypes.c_int),
                ("conv_kernel", ctypes.c_int), ("l2norm_eps", ctypes.c_double),
                ("rmsnorm_eps", ctypes.c_double), ("scale", ctypes.c_double)]


class _Weights(ctypes.Structure):
    _fields_ = [("conv_w", ctypes.POINTER(ctypes.c_double)),
                ("A_log", ctypes.POINTER(ctypes.c_double)),
                ("dt_bias", ctypes.POINTER(ctypes.c_double)),
                ("norm_w", ctypes.POINTER(ctypes.c_double))]


@dataclass(frozen=True)
class Geometry:
    """Per-rank layer geometry: Hk K-heads, Hv V-heads (Hv % Hk == 0)."""
    num_k_heads: int
    num_v_heads: int
    head_k_dim: int
    head_v_dim: int
    conv_kernel: int = 4
    l2norm_eps: float = 1e-6
    rmsnorm_eps: float = 1e-6
    scale: float = 0.0  # <= 0 means 1/sqrt(head_k_dim)

    @property
    def channels(self) -> int:
        return 2 * self.num_k_heads * self.head_k_dim + self.num_v_heads * self.head_v_dim

    def _c(self) -> _Geom:
        return _Geom(self.num_k_heads, self.num_v_heads, self.head_k_dim,
                     self.head_v_dim, self.conv_kernel, self.l2norm_eps,
                     self.rmsnorm_eps, self.scale)


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _dp(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _ip(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int))


class Weights:
    """Layer weights as f64 arrays: conv_w [C][K], A_log [Hv], dt_bias [Hv],
    norm_w [dv]."""

    def __init__(self, conv_w, A_log, dt_bias, norm_w):
        self.conv_w = _f64(conv_w)
        self.A_log = _f64(A_log)
        self.dt_bias = _f64(dt_bias)
        self.norm_w = _f64(norm_w)

    def _c(self) -> _Weights:
        return _Weights(_dp(self.conv_w), _dp(self.A_log), _dp(self.dt_bias),
                        _dp(self.norm_w))


def default_threads() -> int:
    return max(1, min(os.cpu_count() or 1, 16))


def sequences(geom: Geometry, w: Weights, cu_seqlens, x, z, a, b, S0, window0,
              head_mask=None, chunk: int = 0, nthreads: int | None = None):
    """Run N independent sequences (tokens cu[n]..cu[n+1] of the packed
    inputs).  x [T][C], z [T][Hv][dv], a/b [T][Hv], S0 [N][Hv][dk][dv],
    window0 [N][K][C].  Returns (y, o, S, window) as new f64 arrays.  With a
    head mask only the masked heads' y/o/S are meaningful."""
    lib = _load()
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    N = cu.size - 1
    x, z, a, b = _f64(x), _f64(z), _f64(a), _f64(b)
    T = int(cu[-1])
    Hv, dv = geom.num_v_heads, geom.head_v_dim
    S = _f64(S0).copy()
    W = _f64(window0).copy()
    y = np.zeros((T, Hv, dv))
    o = np.zeros((T, Hv, dv))
    mask = None
    if head_mask is not None:
        mask = np.ascontiguousarray(np.asarray(head_mask, dtype=np.uint8))
    g = geom._c()
    wc = w._c()
    rc = lib.ogdn_sequences(ctypes.byref(g), ctypes.byref(wc), N, _ip(cu), _dp(x), _dp(z),
                            _dp(a), _dp(b), _dp(S), _dp(W), _dp(y), _dp(o),
                            mask.ctypes.data if mask is not None else None,
                            int(chunk), nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return y, o, S, W


def pool_run(geom: Geometry, w: Weights, pool_S, pool_conv, cu_seqlens, slot_idx,
             x, z, a, b, has_init=None, nthreads: int | None = None):
    """Slot-pool form (decode: cu = [0, 1, ..., B]; prefill: packed lengths).
    Updates pool_S [P][Hv][dk][dv] and pool_conv [P][K][C] (f64, in place)
    and returns (y, o)."""
    lib = _load()
    assert pool_S.dtype == np.float64 and pool_S.flags.c_contiguous
    assert pool_conv.dtype == np.float64 and pool_conv.flags.c_contiguous
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    sl = np.ascontiguousarray(np.asarray(slot_idx, dtype=np.int32))
    N = cu.size - 1
    T = int(cu[-1])
    x, z, a, b = _f64(x), _f64(z), _f64(a), _f64(b)
    y = np.zeros((T, geom.num_v_heads, geom.head_v_dim))
    o = np.zeros_like(y)
    hi = None
    if has_init is not None:
        hi = np.ascontiguousarray(np.asarray(has_init, dtype=np.uint8))
    g = geom._c()
    wc = w._c()
    rc = lib.ogdn_pool_run(ctypes.byref(g), ctypes.byref(wc), _dp(pool_S), _dp(pool_conv),
                           pool_S.shape[0], N, _ip(cu), _ip(sl),
                           hi.ctypes.data if hi is not None else None,
                           _dp(x), _dp(z), _dp(a), _dp(b), _dp(y), _dp(o),
                           nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return y, o


def linear(x, w):
    """A projection: y[m][n] = sum_k x[m][k] w[n][k], with w stored [out][in]
    like a Linear layer's weight.  These are the in_proj_qkv, in_proj_z,
    in_proj_b, in_proj_a and out_proj products around the layer (cortex commit
    95dc874, TpQwen3_5GatedDeltaNet bullet).  One f64 matrix product."""
    return _f64(x) @ _f64(w).T


@dataclass
class Projections:
    """Projection weights of one block, [out][in] each: qkv [C][H] (output in
    [q | k | v] channel order), z [Hv*dv][H], b [Hv][H], a [Hv][H] and
    out [H][Hv*dv] (cortex commit 95dc874, TpQwen3_5GatedDeltaNet bullet)."""
    qkv: np.ndarray
    z: np.ndarray
    b: np.ndarray
    a: np.ndarray
    out: np.ndarray


def decode_block(geom: Geometry, w: Weights, proj: Projections, pool_S, pool_conv, slot_idx,
                 hidden, nthreads: int | None = None):
    """One decode token per row through the whole block: the four input
    projections of hidden [B][H], the layer on the slot pool (pool_run, which
    updates the pools in place), then out_proj of the gated-norm output
    (cortex commit 95dc874, TpQwen3_5GatedDeltaNet; the batched decode chain
    of pegainfer PR #1003, PR body, batch_decode/prefill bullet).  No rounding
    between the steps.  Returns (out [B][H], inputs, y [B][Hv][dv]) where
    inputs holds the projected x, z, a, b."""
    h = _f64(hidden)
    B = h.shape[0]
    Hv, dv = geom.num_v_heads, geom.head_v_dim
    inp = dict(x=linear(h, proj.qkv), z=linear(h, proj.z).reshape(B, Hv, dv),
               b=linear(h, proj.b), a=linear(h, proj.a))
    y, _ = pool_run(geom, w, pool_S, pool_conv, np.arange(B + 1, dtype=np.int32), slot_idx,
                    inp["x"], inp["z"], inp["a"], inp["b"], nthreads=nthreads)
    return linear(y.reshape(B, Hv * dv), proj.out), inp, y


def compact(geom: Geometry, pool_S, pool_conv, src, dst):
    """Copy slot src[i] to slot dst[i] (state and window), in place."""
    lib = _load()
    s = np.ascontiguousarray(np.asarray(src, dtype=np.int32))
    d = np.ascontiguousarray(np.asarray(dst, dtype=np.int32))
    g = geom._c()
    rc = lib.ogdn_compact(ctypes.byref(g), _dp(pool_S), _dp(pool_conv), pool_S.shape[0],
                          _ip(s), _ip(d), s.size)
    if rc != 0:
        raise ValueError("oracle rejected the arguments")


# ---- single steps, exposed so that tests can pin each one on its own ----

def silu(x: float) -> float:
    return _load().ogdn_silu(float(x))


def softplus(x: float) -> float:
    return _load().ogdn_softplus(float(x))


def gates(A_log: float, dt_bias: float, a: float, b: float):
    g = ctypes.c_double()
    beta = ctypes.c_double()
    _load().ogdn_gates(float(A_log), float(dt_bias), float(a), float(b),
                       ctypes.byref(g), ctypes.byref(beta))
    return g.value, beta.value


def l2norm(x, eps: float = 1e-6, mult: float = 1.0):
    x = _f64(x)
    out = np.empty_like(x)
    _load().ogdn_l2norm(_dp(x), x.size, eps, mult, _dp(out))
    return out


def gdr_step(g: float, beta: float, k, v, q, S):
    """One token on S [dk][dv]; returns (S_new, o)."""
    k, v, q = _f64(k), _f64(v), _f64(q)
    S = _f64(S).copy()
    o = np.empty(v.size)
    _load().ogdn_gdr_step(k.size, v.size, float(g), float(beta), _dp(k), _dp(v), _dp(q),
                          _dp(S), _dp(o))
    return S, o


def gated_rmsnorm(o, z, w, eps: float = 1e-6):
    o, z, w = _f64(o), _f64(z), _f64(w)
    y = np.empty_like(o)
    _load().ogdn_gated_rmsnorm(o.size, _dp(o), _dp(z), _dp(w), eps, _dp(y))
    return y


def conv_silu(conv_w, window, x):
    """Conv + SiLU of every channel.  conv_w [C][K], window [K][C], x [T][C]
    -> [T][C]."""
    lib = _load()
    conv_w, window, x = _f64(conv_w), _f64(window), _f64(x)
    T, C = x.shape
    K = conv_w.shape[1]
    out = np.empty((T, C))
    stream = np.empty(K + T)
    for ch in range(C):
        col = np.empty(T)
        lib.ogdn_conv_channel(C, K, _dp(np.ascontiguousarray(conv_w[ch])), _dp(window),
                              _dp(x), T, ch, _dp(stream), _dp(col), 1)
        out[:, ch] = col
    return out
