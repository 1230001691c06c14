"""MI355X (gfx950) Gated DeltaNet layer core: Python binding of libgdn.so.

The functions below carry the names of the C entry points in include/gdn.h
and only marshal arguments: torch tensors supply device memory and the
current HIP stream, numpy arrays supply host-side index copies.  Every step of
the layer runs in the library's HIP kernels; nothing here computes.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import numpy as np
import torch

from . import _abi
from ._abi import GDN_BF16, GDN_F32, GdnError

__all__ = ["Geometry", "LayerWeights", "StatePool", "GdnError", "gdn_slot_bytes",
           "gdn_prefill_scratch_bytes", "gdn_decode_workspace_bytes", "decode_workspace",
           "gdn_conv_update", "gdn_decode_batch",
           "gdn_decode_step", "gdn_decode_step_noalloc", "gdn_prefill_chunked", "gdn_state_compact", "gdn_check_slots", "gdn_linear",
           "library"]


def library():
    """The loaded libgdn.so (raises ImportError if it is not built)."""
    return _abi.load()


_ACT = {"f32": (GDN_F32, torch.float32), "bf16": (GDN_BF16, torch.bfloat16)}


@dataclass(frozen=True)
class Geometry:
    """Rank-local layer geometry (gdn_geometry)."""
    num_k_heads: int
    num_v_heads: int
    head_k_dim: int
    head_v_dim: int
    conv_kernel: int = 4
    act: str = "bf16"
    l2norm_eps: float = 1e-6
    rmsnorm_eps: float = 1e-6
    scale: float = 0.0

    @property
    def channels(self) -> int:
        return 2 * self.num_k_heads * self.head_k_dim + self.num_v_heads * self.head_v_dim

    @property
    def act_dtype(self) -> torch.dtype:
        return _ACT[self.act][1]

    def c(self) -> _abi.gdn_geometry:
        return _abi.gdn_geometry(self.num_k_heads, self.num_v_heads, self.head_k_dim,
                                 self.head_v_dim, self.conv_kernel, _ACT[self.act][0],
                                 self.l2norm_eps, self.rmsnorm_eps, self.scale)


def _ptr(t: torch.Tensor | None, dtype: torch.dtype | None = None, numel: int | None = None,
         name: str = "tensor") -> int | None:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements, got {t.numel()}")
    return t.data_ptr()


def _host_i32(a, n: int | None = None, name: str = "array"):
    if a is None:
        return None, None
    arr = np.ascontiguousarray(np.asarray(a, dtype=np.int32))
    if n is not None and arr.size != n:
        raise ValueError(f"{name} must have {n} entries")
    return arr, arr.ctypes.data_as(ctypes.c_void_p)


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


class LayerWeights:
    """Device weights of one layer: conv_weight [C][K] (act dtype), A_log [Hv],
    dt_bias [Hv], norm_weight [dv] (f32)."""

    def __init__(self, geom: Geometry, conv_weight, A_log, dt_bias, norm_weight):
        C, K = geom.channels, geom.conv_kernel
        self._keep = (conv_weight, A_log, dt_bias, norm_weight)
        self.c = _abi.gdn_layer_weights(
            _ptr(conv_weight, geom.act_dtype, C * K, "conv_weight"),
            _ptr(A_log, torch.float32, geom.num_v_heads, "A_log"),
            _ptr(dt_bias, torch.float32, geom.num_v_heads, "dt_bias"),
            _ptr(norm_weight, torch.float32, geom.head_v_dim, "norm_weight"))


class StatePool:
    """Slot pool of one layer: recurrent [P][Hv][dk][dv] f32, conv [P][K][C] act."""

    def __init__(self, geom: Geometry, recurrent: torch.Tensor, conv: torch.Tensor):
        P = recurrent.shape[0]
        self.num_slots = P
        self.recurrent, self.conv = recurrent, conv
        per = geom.num_v_heads * geom.head_k_dim * geom.head_v_dim
        self.c = _abi.gdn_state_pool(
            _ptr(recurrent, torch.float32, P * per, "recurrent"),
            _ptr(conv, geom.act_dtype, P * geom.conv_kernel * geom.channels, "conv"), P)


def gdn_slot_bytes(geom: Geometry) -> tuple[int, int]:
    lib = _abi.load()
    r, c = ctypes.c_size_t(), ctypes.c_size_t()
    g = geom.c()
    _abi.check(lib.gdn_slot_bytes(ctypes.byref(g), ctypes.byref(r), ctypes.byref(c)))
    return r.value, c.value


def gdn_prefill_scratch_bytes(geom: Geometry, total_tokens: int, num_seqs: int) -> int:
    lib = _abi.load()
    n = ctypes.c_size_t()
    g = geom.c()
    _abi.check(lib.gdn_prefill_scratch_bytes(ctypes.byref(g), int(total_tokens),
                                             int(num_seqs), ctypes.byref(n)))
    return n.value


def gdn_decode_workspace_bytes(geom: Geometry, B: int) -> int:
    lib = _abi.load()
    n = ctypes.c_size_t()
    g = geom.c()
    _abi.check(lib.gdn_decode_workspace_bytes(ctypes.byref(g), int(B), ctypes.byref(n)))
    return n.value


def decode_workspace(geom: Geometry, B: int, device="cuda") -> torch.Tensor:
    """A zero-filled device workspace for gdn_decode_step calls of up to B
    rows (torch allocates it; the library keeps it zero between calls)."""
    return torch.zeros(max(gdn_decode_workspace_bytes(geom, B), 256), dtype=torch.uint8,
                       device=device)


def gdn_conv_update(geom: Geometry, w: LayerWeights, pool: StatePool, slot_idx: torch.Tensor,
                    qkv_in: torch.Tensor, qkv_out: torch.Tensor, slot_idx_host=None,
                    stream=None) -> None:
    lib = _abi.load()
    B = slot_idx.numel()
    C = geom.channels
    _, host = _host_i32(slot_idx_host, B, "slot_idx_host")
    g = geom.c()
    _abi.check(lib.gdn_conv_update(
        ctypes.byref(g), ctypes.byref(w.c), ctypes.byref(pool.c),
        _ptr(slot_idx, torch.int32, B, "slot_idx"), host, B,
        _ptr(qkv_in, geom.act_dtype, B * C, "qkv_in"),
        _ptr(qkv_out, torch.float32, B * C, "qkv_out"), _stream(stream)))


def gdn_decode_batch(geom: Geometry, w: LayerWeights, pool: StatePool, slot_idx: torch.Tensor,
                     qkv: torch.Tensor, z: torch.Tensor, a: torch.Tensor, b: torch.Tensor,
                     y: torch.Tensor, o_raw: torch.Tensor | None = None, slot_idx_host=None,
                     stream=None) -> None:
    lib = _abi.load()
    B = slot_idx.numel()
    Hv, dv = geom.num_v_heads, geom.head_v_dim
    act = geom.act_dtype
    _, host = _host_i32(slot_idx_host, B, "slot_idx_host")
    g = geom.c()
    _abi.check(lib.gdn_decode_batch(
        ctypes.byref(g), ctypes.byref(w.c), ctypes.byref(pool.c),
        _ptr(slot_idx, torch.int32, B, "slot_idx"), host, B,
        _ptr(qkv, torch.float32, B * geom.channels, "qkv"),
        _ptr(z, act, B * Hv * dv, "z"), _ptr(a, act, B * Hv, "a"), _ptr(b, act, B * Hv, "b"),
        _ptr(y, act, B * Hv * dv, "y"), _ptr(o_raw, torch.float32, B * Hv * dv, "o_raw"),
        _stream(stream)))


def gdn_decode_step(geom: Geometry, w: LayerWeights, pool: StatePool, slot_idx: torch.Tensor,
                    qkv_in: torch.Tensor, z: torch.Tensor, a: torch.Tensor, b: torch.Tensor,
                    y: torch.Tensor, workspace: torch.Tensor, o_raw: torch.Tensor | None = None,
                    slot_idx_host=None, stream=None) -> None:
    """workspace: a uint8 device tensor from decode_workspace (zero-filled
    before first use, left zero-filled by every call)."""
    lib = _abi.load()
    B = slot_idx.numel()
    Hv, dv = geom.num_v_heads, geom.head_v_dim
    act = geom.act_dtype
    _, host = _host_i32(slot_idx_host, B, "slot_idx_host")
    if workspace is not None and workspace.dtype != torch.uint8:
        raise ValueError("workspace must be a uint8 tensor")
    g = geom.c()
    _abi.check(lib.gdn_decode_step(
        ctypes.byref(g), ctypes.byref(w.c), ctypes.byref(pool.c),
        _ptr(slot_idx, torch.int32, B, "slot_idx"), host, B,
        _ptr(qkv_in, act, B * geom.channels, "qkv_in"),
        _ptr(z, act, B * Hv * dv, "z"), _ptr(a, act, B * Hv, "a"), _ptr(b, act, B * Hv, "b"),
        _ptr(y, act, B * Hv * dv, "y"), _ptr(o_raw, torch.float32, B * Hv * dv, "o_raw"),
        _ptr(workspace, name="workspace"), workspace.numel() if workspace is not None else 0,
        _stream(stream)))


def gdn_decode_step_noalloc(geom: Geometry, w: LayerWeights, pool: StatePool,
                            slot_idx: torch.Tensor, qkv_in: torch.Tensor, z: torch.Tensor,
                            a: torch.Tensor, b: torch.Tensor, y: torch.Tensor,
                            o_raw: torch.Tensor | None = None, slot_idx_host=None,
                            stream=None) -> None:
    """gdn_decode_step with the library-held workspace (no workspace argument;
    calls on one GPU must not overlap in time)."""
    lib = _abi.load()
    B = slot_idx.numel()
    Hv, dv = geom.num_v_heads, geom.head_v_dim
    act = geom.act_dtype
    _, host = _host_i32(slot_idx_host, B, "slot_idx_host")
    g = geom.c()
    _abi.check(lib.gdn_decode_step_noalloc(
        ctypes.byref(g), ctypes.byref(w.c), ctypes.byref(pool.c),
        _ptr(slot_idx, torch.int32, B, "slot_idx"), host, B,
        _ptr(qkv_in, act, B * geom.channels, "qkv_in"),
        _ptr(z, act, B * Hv * dv, "z"), _ptr(a, act, B * Hv, "a"), _ptr(b, act, B * Hv, "b"),
        _ptr(y, act, B * Hv * dv, "y"), _ptr(o_raw, torch.float32, B * Hv * dv, "o_raw"),
        _stream(stream)))


def gdn_prefill_chunked(geom: Geometry, w: LayerWeights, pool: StatePool, cu_seqlens_host,
                        cu_seqlens: torch.Tensor, slot_idx: torch.Tensor, qkv_in: torch.Tensor,
                        z: torch.Tensor, a: torch.Tensor, b: torch.Tensor, y: torch.Tensor,
                        scratch: torch.Tensor, o_raw: torch.Tensor | None = None,
                        has_init: torch.Tensor | None = None, slot_idx_host=None,
                        stream=None) -> None:
    lib = _abi.load()
    cu_h, cu_hp = _host_i32(cu_seqlens_host, None, "cu_seqlens_host")
    N = cu_h.size - 1
    T = int(cu_h[-1]) if N >= 0 else 0
    Hv, dv = geom.num_v_heads, geom.head_v_dim
    act = geom.act_dtype
    _, host = _host_i32(slot_idx_host, N, "slot_idx_host")
    if scratch is not None and scratch.dtype != torch.uint8:
        raise ValueError("scratch must be a uint8 tensor")
    g = geom.c()
    _abi.check(lib.gdn_prefill_chunked(
        ctypes.byref(g), ctypes.byref(w.c), ctypes.byref(pool.c), cu_hp,
        _ptr(cu_seqlens, torch.int32, N + 1, "cu_seqlens"),
        _ptr(slot_idx, torch.int32, N, "slot_idx"), host,
        _ptr(has_init, torch.uint8, N, "has_init"), N,
        _ptr(qkv_in, act, T * geom.channels, "qkv_in"), _ptr(z, act, T * Hv * dv, "z"),
        _ptr(a, act, T * Hv, "a"), _ptr(b, act, T * Hv, "b"), _ptr(y, act, T * Hv * dv, "y"),
        _ptr(o_raw, torch.float32, T * Hv * dv, "o_raw"), _ptr(scratch, name="scratch"),
        scratch.numel() if scratch is not None else 0, _stream(stream)))


def gdn_state_compact(geom: Geometry, pools: list[StatePool], src_host, dst_host,
                      src: torch.Tensor, dst: torch.Tensor, stream=None) -> None:
    lib = _abi.load()
    s_h, s_hp = _host_i32(src_host, None, "src_host")
    n = s_h.size
    _, d_hp = _host_i32(dst_host, n, "dst_host")
    arr = (_abi.gdn_state_pool * max(len(pools), 1))(*[p.c for p in pools])
    g = geom.c()
    _abi.check(lib.gdn_state_compact(
        ctypes.byref(g), arr, len(pools), s_hp, d_hp, _ptr(src, torch.int32, n, "src"),
        _ptr(dst, torch.int32, n, "dst"), n, _stream(stream)))


def gdn_check_slots(slot_idx: torch.Tensor, num_slots: int, result: torch.Tensor,
                    stream=None) -> None:
    """Enqueue the device-side check of slot_idx; result (int32 device [2])
    receives (status, smallest offending row or INT32_MAX)."""
    lib = _abi.load()
    B = slot_idx.numel()
    _abi.check(lib.gdn_check_slots(_ptr(slot_idx, torch.int32, B, "slot_idx"), B,
                                   int(num_slots), _ptr(result, torch.int32, 2, "result"),
                                   _stream(stream)))


def _rows(t: torch.Tensor, name: str) -> tuple[int, int, int]:
    """(rows, cols, row stride) of a 2-D bf16 device tensor with unit column stride."""
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != torch.bfloat16 or t.dim() != 2:
        raise ValueError(f"{name} must be a 2-D bfloat16 tensor")
    if t.stride(1) != 1 and t.size(1) > 1:
        raise ValueError(f"{name} must have unit column stride")
    return t.size(0), t.size(1), t.stride(0) if t.size(0) > 1 else t.size(1)


def gdn_linear(x: torch.Tensor, outs, stream=None) -> None:
    """outs: 1..4 pairs (weight [N][K], out [M][N]); each out = x @ weight^T.
    x and out may be row-strided views (unit column stride); weights are dense."""
    lib = _abi.load()
    M, K, ldx = _rows(x, "x")
    arr = (_abi.gdn_linear_out * max(len(outs), 1))()
    for i, (w, y) in enumerate(outs):
        N, Kw, _ = _rows(w, f"weight {i}")
        if not w.is_contiguous() or Kw != K:
            raise ValueError(f"weight {i} must be a dense [N][{K}] tensor")
        My, Ny, ldy = _rows(y, f"out {i}")
        if My != M or Ny != N:
            raise ValueError(f"out {i} must be [{M}][{N}]")
        arr[i] = _abi.gdn_linear_out(w.data_ptr(), y.data_ptr(), N, ldy)
    _abi.check(lib.gdn_linear(x.data_ptr(), M, K, ldx, arr, len(outs), _stream(stream)))
