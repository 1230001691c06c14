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


def fused_step(L: Layer, P: Pool, slot_idx, x, z, a, b, workspace=None, with_host=True,
               want_o=True, stream=None):
    """gdn_decode_step (conv, state step and gated norm in one launch);
    returns (y, o_raw).  A fresh zero-filled workspace unless one is given."""
    s = L.s
    B = len(slot_idx)
    ad = act_dtype(s)
    hs = np.asarray(slot_idx, np.int32)
    y = torch.empty(B, s.num_v_heads, s.head_v_dim, device=DEV, dtype=ad)
    o = torch.empty(B, s.num_v_heads, s.head_v_dim, device=DEV) if want_o else None
    ws = gdn.decode_workspace(L.geom, B) if workspace is None else workspace
    xd, zd, ad_, bd = dev(x, ad), dev(z, ad), dev(a, ad), dev(b, ad)
    sl = dev(hs, torch.int32)
    if stream is not None:   # the inputs were copied on the current stream
        stream.wait_stream(torch.cuda.current_stream())
        for t in (xd, zd, ad_, bd, sl, y) + ((o,) if o is not None else ()):
            t.record_stream(stream)   # not reused before that stream is done
    gdn.gdn_decode_step(L.geom, L.w, P.pool, sl, xd, zd, ad_, bd, y, ws, o_raw=o,
                        slot_idx_host=hs if with_host else None, stream=stream)
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


class ServingRows:
    """Bookkeeping of a decode schedule (tests only): logical rows, each
    starting from a pool slot's initial state or, when admitted later, from
    zeros; the tokens each row has seen and its last-layer y per token; and
    the slot it sits in, which changes when retired rows' slots are compacted
    by hole filling (workloads.retire_plan: survivors move into the prefix,
    admitted rows take the slots behind them)."""

    def __init__(self, slots0):
        self.rows = [dict(start=int(sl), toks=[]) for sl in slots0]
        self.active = list(range(len(slots0)))
        self.slot_of = {i: int(sl) for i, sl in enumerate(slots0)}

    def live_slots(self) -> np.ndarray:
        return np.array([self.slot_of[i] for i in self.active], np.int32)

    def retire(self, rng, P: int, n_admit: int | None = None):
        """Retire a seeded half, compact, admit n_admit new rows (default: as
        many as retired).  Returns (src, dst, admitted slots); the caller
        runs the compaction and zeroes the admitted slots."""
        import workloads as wl
        keep, new_slots, src, dst = wl.retire_plan(rng, self.live_slots(), P)
        survivors = [i for i, k in zip(self.active, keep) if k]
        for i, ns in zip(survivors, new_slots):
            self.slot_of[i] = int(ns)
        n_new = len(self.active) - len(survivors) if n_admit is None else n_admit
        free = list(range(len(survivors), len(survivors) + n_new))
        for f in free:
            self.rows.append(dict(start=None, toks=[]))
            self.slot_of[len(self.rows) - 1] = f
        self.active = survivors + list(range(len(self.rows) - n_new, len(self.rows)))
        return src, dst, free

    def record(self, inp: dict, y_host: np.ndarray) -> None:
        """Row j of this step's inputs (and of the last layer's y) belongs to
        the j-th active row."""
        for j, i in enumerate(self.active):
            self.rows[i]["toks"].append({k: inp[k][j] for k in ("x", "z", "a", "b")}
                                        | {"y": y_host[j]})

    def check(self, Ls, Ps, init, s, tag=""):
        """Every live row against the oracle running its tokens as one
        sequence per layer (layers share each step's inputs): every layer's
        state (f32 bar) and conv window (bit-exact), the last layer's y."""
        act = self.active
        lens = [len(self.rows[i]["toks"]) for i in act]
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        tok = {k: np.concatenate([np.stack([t[k] for t in self.rows[i]["toks"]]) for i in act])
               for k in ("x", "z", "a", "b", "y")}
        slots = self.live_slots()
        shape_s = (len(act), s.num_v_heads, s.head_k_dim, s.head_v_dim)
        for l, (L, P) in enumerate(zip(Ls, Ps)):
            S0 = np.zeros(shape_s)
            W0 = np.zeros((len(act), s.conv_kernel, s.channels))
            for n, i in enumerate(act):
                st = self.rows[i]["start"]
                if st is not None:
                    S0[n] = init[l][0][st]
                    W0[n] = init[l][1][st]
            yo, _, Sn, Wn = oracle.sequences(L.og, L.ow, cu, tok["x"], tok["z"], tok["a"],
                                             tok["b"], S0, W0)
            del S0
            assert_close(f"{tag} layer {l} states of {len(act)} live rows",
                         maxrel_states(host(P.rec)[slots], Sn), TOL_F32)
            np.testing.assert_array_equal(host(P.conv)[slots], Wn,
                                          err_msg=f"{tag} layer {l} conv windows")
            if l == len(Ls) - 1:
                assert_close(f"{tag} last-layer y", maxrel_heads(tok["y"], yo), y_tol(s))
