"""Shared plumbing of the GPU parity tests: device copies of seeded inputs,
calls through the C ABI, and the comparison metrics.

Tolerances (the layer's parity bar):
  * bf16 outputs (y):            per-V-head max-rel <= 2e-2
  * f32 state and f32 outputs:   per-(slot, V-head) / per-V-head max-rel <= 1e-3
max-rel of x against reference r over a group = max|x - r| / max|r|; an
element-wise ratio is ill-conditioned where q.k ~ 0 makes o tiny.
"""
from __future__ import annotations

import numpy as np
import torch

import linear_attention_causal_amd as gdn
import oracle
from workloads import Shape

TOL_BF16 = 2e-2
TOL_F32 = 1e-3

DEV = "cuda"


def geometry(s: Shape) -> gdn.Geometry:
    return gdn.Geometry(s.num_k_heads, s.num_v_heads, s.head_k_dim, s.head_v_dim,
                        s.conv_kernel, s.act)


def ogeometry(s: Shape) -> oracle.Geometry:
    return oracle.Geometry(s.num_k_heads, s.num_v_heads, s.head_k_dim, s.head_v_dim,
                           s.conv_kernel)


def act_dtype(s: Shape):
    return torch.bfloat16 if s.act == "bf16" else torch.float32


def dev(x, dtype=torch.float32) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV).to(dtype).contiguous()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


class Layer:
    """Device weights of one layer plus the matching oracle weights."""

    def __init__(self, s: Shape, w: dict):
        self.s = s
        self.geom = geometry(s)
        self.t = dict(conv_w=dev(w["conv_w"], act_dtype(s)), A_log=dev(w["A_log"]),
                      dt_bias=dev(w["dt_bias"]), norm_w=dev(w["norm_w"]))
        self.w = gdn.LayerWeights(self.geom, self.t["conv_w"], self.t["A_log"],
                                  self.t["dt_bias"], self.t["norm_w"])
        self.ow = oracle.Weights(w["conv_w"], w["A_log"], w["dt_bias"], w["norm_w"])
        self.og = ogeometry(s)


class Pool:
    def __init__(self, s: Shape, rec: np.ndarray, conv: np.ndarray):
        self.rec = dev(rec)
        self.conv = dev(conv, act_dtype(s))
        self.pool = gdn.StatePool(geometry(s), self.rec, self.conv)


def decode_step(L: Layer, P: Pool, slot_idx, x, z, a, b, with_host=True, want_o=True):
    """conv_update + decode_batch for one token per row; returns (y, o_raw)."""
    s = L.s
    B = len(slot_idx)
    sl = dev(np.asarray(slot_idx, np.int32), torch.int32)
    qkv = torch.empty(B, s.channels, device=DEV, dtype=torch.float32)
    y = torch.empty(B, s.num_v_heads, s.head_v_dim, device=DEV, dtype=act_dtype(s))
    o = torch.empty(B, s.num_v_heads, s.head_v_dim, device=DEV) if want_o else None
    hs = np.asarray(slot_idx, np.int32) if with_host else None
    gdn.gdn_conv_update(L.geom, L.w, P.pool, sl, dev(x, act_dtype(s)), qkv, slot_idx_host=hs)
    gdn.gdn_decode_batch(L.geom, L.w, P.pool, sl, qkv, dev(z, act_dtype(s)),
                         dev(a, act_dtype(s)), dev(b, act_dtype(s)), y, o, slot_idx_host=hs)
    return y, o


def prefill(L: Layer, P: Pool, cu, slot_idx, x, z, a, b, has_init=None, want_o=True):
    s = L.s
    cu = np.asarray(cu, np.int32)
    T = int(cu[-1])
    N = cu.size - 1
    y = torch.empty(T, s.num_v_heads, s.head_v_dim, device=DEV, dtype=act_dtype(s))
    o = torch.empty(T, s.num_v_heads, s.head_v_dim, device=DEV) if want_o else None
    nbytes = gdn.gdn_prefill_scratch_bytes(L.geom, T, N)
    scratch = torch.empty(max(nbytes, 256), device=DEV, dtype=torch.uint8)
    hi = dev(np.asarray(has_init, np.uint8), torch.uint8) if has_init is not None else None
    gdn.gdn_prefill_chunked(L.geom, L.w, P.pool, cu, dev(cu, torch.int32),
                            dev(np.asarray(slot_idx, np.int32), torch.int32),
                            dev(x, act_dtype(s)), dev(z, act_dtype(s)), dev(a, act_dtype(s)),
                            dev(b, act_dtype(s)), y, scratch, o_raw=o, has_init=hi,
                            slot_idx_host=np.asarray(slot_idx, np.int32))
    return y, o


def maxrel_heads(x: np.ndarray, r: np.ndarray, head_axis: int = -2) -> np.ndarray:
    """Per-V-head max|x - r| / max|r| (x, r [..., Hv, dv])."""
    x = np.moveaxis(np.asarray(x, np.float64), head_axis, 0)
    r = np.moveaxis(np.asarray(r, np.float64), head_axis, 0)
    H = x.shape[0]
    err = np.abs(x - r).reshape(H, -1).max(1)
    ref = np.abs(r).reshape(H, -1).max(1)
    return err / np.maximum(ref, 1e-30)


def maxrel_states(x: np.ndarray, r: np.ndarray) -> np.ndarray:
    """Per-(slot, V-head) max-rel of states [..., Hv, dk, dv] -> [..., Hv]."""
    x = np.asarray(x, np.float64)
    r = np.asarray(r, np.float64)
    err = np.abs(x - r).max(axis=(-1, -2))
    ref = np.abs(r).max(axis=(-1, -2))
    return err / np.maximum(ref, 1e-30)


def assert_close(name, rel, tol):
    worst = float(np.max(rel)) if np.size(rel) else 0.0
    print(f"  {name}: max-rel {worst:.3e} (tol {tol:.0e})", flush=True)
    assert worst <= tol, f"{name}: max-rel {worst:.3e} > {tol:.0e}"


def y_tol(s: Shape) -> float:
    return TOL_BF16 if s.act == "bf16" else TOL_F32
