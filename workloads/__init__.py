"""Seeded synthetic inputs for the Gated DeltaNet layer.

This module only draws numbers and rounds them to their storage type; it holds
none of the layer's arithmetic.  Both the GPU path (through the tests and the
benchmark) and the CPU oracle consume exactly the arrays it returns.

Recipe: numpy PCG64 `default_rng(seed)`; every value is drawn in float64, cast
to float32 and, for bf16 activations, rounded to bfloat16 (round to nearest
even).  Arrays come back as float32 numpy arrays whose values are exactly
representable in the activation dtype.  N(m, s) means mean m, standard
deviation s.

Distributions (all workloads):
  fused [q|k|v] input x, z, a, b ~ N(0, 1)
  A_log = log U(1, 16) per V-head          (slow-decay variant: log U(0.002, 0.03))
  dt_bias ~ U(-1, 1) per V-head
  conv weight ~ N(0, 0.25)
  norm weight = 1 + 0.1 N(0, 1)
  initial recurrent / conv states ~ N(0, 0.1) where a workload asks for them.
  block workloads: hidden rows ~ N(0, 1); projection weights ~ N(0, 1/in)
  in bf16, so the projected x, z, a, b are again about N(0, 1).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Shape:
    num_k_heads: int
    num_v_heads: int
    head_k_dim: int
    head_v_dim: int
    conv_kernel: int = 4
    act: str = "bf16"  # "bf16" or "f32"

    @property
    def channels(self) -> int:
        return 2 * self.num_k_heads * self.head_k_dim + self.num_v_heads * self.head_v_dim


def round_bf16(x) -> np.ndarray:
    """float -> nearest bfloat16 (ties to even), returned as float32."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).reshape(x.shape)


def to_act(x, act: str) -> np.ndarray:
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    return round_bf16(x32) if act == "bf16" else x32


def _normal(rng, size, std, act):
    return to_act(rng.standard_normal(size) * std, act)


def layer_weights(rng, s: Shape, slow_decay: bool = False) -> dict:
    C, K, Hv = s.channels, s.conv_kernel, s.num_v_heads
    conv_w = _normal(rng, (C, K), 0.25, s.act)
    lo, hi = (0.002, 0.03) if slow_decay else (1.0, 16.0)
    A_log = np.log(rng.uniform(lo, hi, Hv)).astype(np.float32)
    dt_bias = rng.uniform(-1.0, 1.0, Hv).astype(np.float32)
    norm_w = (1.0 + 0.1 * rng.standard_normal(s.head_v_dim)).astype(np.float32)
    return dict(conv_w=conv_w, A_log=A_log, dt_bias=dt_bias, norm_w=norm_w)


def token_inputs(rng, s: Shape, T: int) -> dict:
    """x [T][C] (fused [q|k|v] before the conv), z [T][Hv][dv], a, b [T][Hv]."""
    x = _normal(rng, (T, s.channels), 1.0, s.act)
    z = _normal(rng, (T, s.num_v_heads, s.head_v_dim), 1.0, s.act)
    a = _normal(rng, (T, s.num_v_heads), 1.0, s.act)
    b = _normal(rng, (T, s.num_v_heads), 1.0, s.act)
    return dict(x=x, z=z, a=a, b=b)


def state_pool(rng, s: Shape, P: int, std: float = 0.1, zero: bool = False):
    """Recurrent pool [P][Hv][dk][dv] float32 and conv pool [P][K][C] (act)."""
    rec_shape = (P, s.num_v_heads, s.head_k_dim, s.head_v_dim)
    conv_shape = (P, s.conv_kernel, s.channels)
    if zero:
        return np.zeros(rec_shape, np.float32), np.zeros(conv_shape, np.float32)
    rec = (rng.standard_normal(rec_shape, dtype=np.float32) * np.float32(std))
    conv = _normal(rng, conv_shape, std, s.act)
    return rec, conv


def bf16_normal(rng, shape, std: float = 1.0) -> np.ndarray:
    """N(0, std) rounded to bfloat16 (float32 array)."""
    return _normal(rng, shape, std, "bf16")


def projection_weights(rng, s: Shape, hidden: int) -> dict:
    """[out][in] bf16 weights: qkv [C][H], z [Hv*dv][H], b, a [Hv][H],
    out [H][Hv*dv].  Draw order: qkv, z, b, a, out."""
    vd = s.num_v_heads * s.head_v_dim
    return dict(qkv=bf16_normal(rng, (s.channels, hidden), hidden ** -0.5),
                z=bf16_normal(rng, (vd, hidden), hidden ** -0.5),
                b=bf16_normal(rng, (s.num_v_heads, hidden), hidden ** -0.5),
                a=bf16_normal(rng, (s.num_v_heads, hidden), hidden ** -0.5),
                out=bf16_normal(rng, (hidden, vd), vd ** -0.5))


# ------------------------------------------------------------- workloads

TINY = Shape(2, 4, 32, 32, 4, "f32")
RANK_LOCAL = Shape(8, 16, 128, 128, 4, "bf16")   # one rank of a two-way split
FULL_HEADS = Shape(16, 32, 128, 128, 4, "bf16")


@dataclass
class Workload:
    name: str
    shape: Shape
    seed: int
    data: dict = field(default_factory=dict)


def tiny(seed: int = 0, T: int = 64, decode_steps: int = 8,
         slow_decay: bool = False) -> Workload:
    """Tiny f32 layer: one sequence, T-token prefill then `decode_steps` decode
    steps; Hk=2, Hv=4, dk=dv=32, K=4; zero initial state in slot 0.
    Draw order: weights, prefill tokens, then one token per decode step."""
    s = TINY
    rng = np.random.default_rng(seed)
    w = layer_weights(rng, s, slow_decay)
    pre = token_inputs(rng, s, T)
    steps = [token_inputs(rng, s, 1) for _ in range(decode_steps)]
    rec, conv = state_pool(rng, s, 1, zero=True)
    return Workload("tiny_f32_t64_d8", s, seed,
                    dict(weights=w, prefill=pre, steps=steps, rec=rec, conv=conv,
                         cu_seqlens=np.array([0, T], np.int32),
                         slot_idx=np.array([0], np.int32)))


def decode_batch(seed: int = 0, B: int = 16, P: int = 64, s: Shape = RANK_LOCAL,
                 slow_decay: bool = False) -> Workload:
    """Batched decode, one layer: B rows drawn without replacement from a pool of
    P slots whose recurrent and conv states are N(0, 0.1).
    Draw order: weights, pools, slot_idx, token inputs."""
    rng = np.random.default_rng(seed)
    w = layer_weights(rng, s, slow_decay)
    rec, conv = state_pool(rng, s, P)
    slot_idx = rng.choice(P, B, replace=False).astype(np.int32)
    inp = token_inputs(rng, s, B)
    return Workload(f"decode_b{B}_hk{s.num_k_heads}_hv{s.num_v_heads}_d{s.head_k_dim}_p{P}",
                    s, seed, dict(weights=w, rec=rec, conv=conv, slot_idx=slot_idx, **inp))


def prefill_single(seed: int = 0, T: int = 4096, s: Shape = RANK_LOCAL,
                   slow_decay: bool = False) -> Workload:
    """One sequence of T tokens, recurrent initial state N(0, 0.1) in slot 0,
    zero conv window.  Draw order: weights, initial state, token inputs."""
    rng = np.random.default_rng(seed)
    w = layer_weights(rng, s, slow_decay)
    rec = (rng.standard_normal((1, s.num_v_heads, s.head_k_dim, s.head_v_dim),
                               dtype=np.float32) * np.float32(0.1))
    conv = np.zeros((1, s.conv_kernel, s.channels), np.float32)
    inp = token_inputs(rng, s, T)
    return Workload(f"prefill_t{T}_hk{s.num_k_heads}_hv{s.num_v_heads}_d{s.head_k_dim}",
                    s, seed, dict(weights=w, rec=rec, conv=conv,
                                  cu_seqlens=np.array([0, T], np.int32),
                                  slot_idx=np.array([0], np.int32),
                                  has_init=np.array([1], np.uint8), **inp))


def prefill_varlen(seed: int = 0, n_seqs: int = 8, lo: int = 128, hi: int = 8192,
                   s: Shape = FULL_HEADS, slow_decay: bool = False,
                   lens=None) -> Workload:
    """Packed varlen prefill: n_seqs lengths U{lo..hi} (inclusive) via
    cu_seqlens, each with its own slot holding N(0, 0.1) recurrent and conv
    states.  Draw order: lengths, weights, pools, token inputs."""
    rng = np.random.default_rng(seed)
    if lens is None:
        lens = rng.integers(lo, hi, endpoint=True, size=n_seqs)
    lens = np.asarray(lens, np.int64)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    w = layer_weights(rng, s, slow_decay)
    rec, conv = state_pool(rng, s, len(lens))
    inp = token_inputs(rng, s, int(cu[-1]))
    return Workload(f"varlen{len(lens)}_hk{s.num_k_heads}_hv{s.num_v_heads}_d{s.head_k_dim}",
                    s, seed, dict(weights=w, rec=rec, conv=conv, cu_seqlens=cu,
                                  slot_idx=np.arange(len(lens), dtype=np.int32),
                                  has_init=np.ones(len(lens), np.uint8), **inp))


def retire_plan(rng, live_slots: np.ndarray, P: int):
    """Retire a seeded half of the live rows and compact by hole filling: the
    surviving rows that sit at or above the new live count move down into the
    free slots below it.  Returns (keep mask over live_slots, the survivors'
    new slots in the same order, src, dst).  Index bookkeeping only; src and
    dst never overlap and dst entries are distinct."""
    live = np.asarray(live_slots, np.int64)
    n = live.size
    keep_mask = np.zeros(n, bool)
    keep_mask[rng.choice(n, n - n // 2, replace=False)] = True
    kept = live[keep_mask]
    n_keep = kept.size
    holes = sorted(set(range(n_keep)) - set(kept.tolist()))
    movers = sorted(int(s) for s in kept if s >= n_keep)
    assert len(holes) == len(movers)
    remap = dict(zip(movers, holes))
    new_slots = np.array([remap.get(int(s), int(s)) for s in kept], np.int32)
    return keep_mask, new_slots, np.array(movers, np.int32), np.array(holes, np.int32)


# Hidden size of the block around the layer.  The pages give none; 2048 is the
# published hidden size of Qwen3-Next, whose linear-attention layers have the
# FULL_HEADS head counts (RANK_LOCAL is one rank of a two-way split of it).
HIDDEN = 2048


def decode_block(seed: int = 0, B: int = 16, P: int = 64, s: Shape = RANK_LOCAL,
                 hidden: int = HIDDEN) -> Workload:
    """One decode token per row through the whole block (input projections,
    layer, out_proj): B rows drawn without replacement from P slots whose
    states are N(0, 0.1); hidden rows [B][H].
    Draw order: layer weights, projection weights, pools, slot_idx, hidden."""
    if s.act != "bf16":
        raise ValueError("the block runs on bf16 activations")
    rng = np.random.default_rng(seed)
    w = layer_weights(rng, s)
    proj = projection_weights(rng, s, hidden)
    rec, conv = state_pool(rng, s, P)
    slot_idx = rng.choice(P, B, replace=False).astype(np.int32)
    h = bf16_normal(rng, (B, hidden))
    return Workload(f"block_b{B}_h{hidden}_hk{s.num_k_heads}_hv{s.num_v_heads}_d{s.head_k_dim}",
                    s, seed, dict(weights=w, proj=proj, rec=rec, conv=conv, slot_idx=slot_idx,
                                  hidden=h))
