"""GPU parity of the projections around the layer (gdn_linear) and of a whole
decode block (input projections, gdn_decode_step, out_proj) against the f64
oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import linear_attention_causal_amd as gdn
import oracle
import workloads as wl
from gpu_helpers import (DEV, TOL_BF16, TOL_F32, Layer, Pool, assert_close, dev, host,
                         maxrel_heads, maxrel_states)

pytestmark = pytest.mark.gpu


def maxrel_rows(x: np.ndarray, r: np.ndarray) -> np.ndarray:
    """Per-row max|x - r| / max|r| of [M][N] arrays; a row whose reference is
    all zero must be exactly zero (reported as 0 or inf)."""
    x = np.asarray(x, np.float64)
    r = np.asarray(r, np.float64)
    err = np.abs(x - r).max(1)
    ref = np.abs(r).max(1)
    return np.where(ref > 0, err / np.where(ref > 0, ref, 1.0), np.where(err > 0, np.inf, 0.0))


def _run_linear(M, K, Ns, seed, x_pad=0, y_pad=0):
    """x [M][K] inside a [M][K + x_pad] buffer; output i [M][N_i] inside a
    [M][N_i + y_pad] buffer whose extra columns hold a canary."""
    print(f"[linear] M={M} K={K} N={Ns} x_pad={x_pad} y_pad={y_pad} seed={seed}", flush=True)
    rng = np.random.default_rng(seed)
    x = wl.bf16_normal(rng, (M, K))
    ws = [wl.bf16_normal(rng, (N, K), K ** -0.5) for N in Ns]
    xb = torch.zeros(M, K + x_pad, device=DEV, dtype=torch.bfloat16)
    xb[:, :K] = dev(x, torch.bfloat16)
    wd = [dev(w, torch.bfloat16) for w in ws]
    canary = -7.0
    yb = [torch.full((M, N + y_pad), canary, device=DEV, dtype=torch.bfloat16) for N in Ns]
    gdn.gdn_linear(xb[:, :K], [(w, y[:, :N]) for w, y, N in zip(wd, yb, Ns)])
    torch.cuda.synchronize()
    for i, (w, y, N) in enumerate(zip(ws, yb, Ns)):
        got = host(y)
        assert_close(f"y{i}", maxrel_rows(got[:, :N], oracle.linear(x, w)), TOL_BF16)
        assert (got[:, N:] == canary).all(), "columns past N were written"


@pytest.mark.parametrize("M,K,Ns", [
    (16, 2048, [4096, 2048, 16, 16]),     # rank-local input projections of 16 decode rows
    (16, 2048, [2048]),                   # rank-local out_proj
    (256, 2048, [8192, 4096, 32, 32]),    # full-head input projections of 256 rows
    (256, 4096, [2048]),                  # full-head out_proj
    (1, 8, [1]),                          # smallest
    (20, 200, [40, 8]),                   # two row tiles, K not a multiple of 32, ragged N
    (37, 96, [24, 17, 16, 3]),            # four row tiles, partial last block
    (100, 32, [100]),                     # K of one step: three waves have no work
    (64, 200, [40, 8]),                   # tiled, K not a multiple of 32
    (130, 72, [200, 5]),                  # tiled, partial row block and K tail
    (512, 1024, [1024]),                  # tiled, large tile
    (300, 200, [16000, 7]),               # 128 x 128 tile: partial row tile, K tail, ragged N
    (300, 232, [16000, 7]),               # 128 x 128 tile: K ends in a stage's second k-step
    (260, 96, [16384]),                   # 128 x 128 tile: fewer k-step stages than loads ahead
])
def test_linear(M, K, Ns):
    _run_linear(M, K, Ns, seed=M + K)


def test_linear_strided_rows():
    """x and the outputs are row-strided views of wider buffers."""
    _run_linear(24, 128, [48, 16], seed=5, x_pad=40, y_pad=24)


def test_linear_empty_rows():
    x = torch.empty(0, 64, device=DEV, dtype=torch.bfloat16)
    w = torch.ones(32, 64, device=DEV, dtype=torch.bfloat16)
    y = torch.empty(0, 32, device=DEV, dtype=torch.bfloat16)
    gdn.gdn_linear(x, [(w, y)])
    torch.cuda.synchronize()


def test_linear_rejects_overlap():
    x = torch.zeros(16, 64, device=DEV, dtype=torch.bfloat16)
    w = torch.zeros(32, 64, device=DEV, dtype=torch.bfloat16)
    with pytest.raises(gdn.GdnError):
        gdn.gdn_linear(x, [(w, x[:, :32])])


# ------------------------------------------------------------------ whole block

def _block_gpu(L, P, proj_d, slots, hidden, s, H):
    """Input projections (one launch), fused decode step, out_proj."""
    B = hidden.shape[0]
    C, vd, Hv = s.channels, s.num_v_heads * s.head_v_dim, s.num_v_heads
    bf = torch.bfloat16
    qkv = torch.empty(B, C, device=DEV, dtype=bf)
    z = torch.empty(B, vd, device=DEV, dtype=bf)
    b = torch.empty(B, Hv, device=DEV, dtype=bf)
    a = torch.empty(B, Hv, device=DEV, dtype=bf)
    y = torch.empty(B, Hv, s.head_v_dim, device=DEV, dtype=bf)
    out = torch.empty(B, H, device=DEV, dtype=bf)
    h = dev(hidden, bf)
    sl = dev(np.asarray(slots, np.int32), torch.int32)
    gdn.gdn_linear(h, [(proj_d["qkv"], qkv), (proj_d["z"], z), (proj_d["b"], b),
                       (proj_d["a"], a)])
    gdn.gdn_decode_step(L.geom, L.w, P.pool, sl, qkv, z, a, b, y,
                        gdn.decode_workspace(L.geom, B),
                        slot_idx_host=np.asarray(slots, np.int32))
    gdn.gdn_linear(y.view(B, vd), [(proj_d["out"], out)])
    torch.cuda.synchronize()
    return dict(x=host(qkv), z=host(z).reshape(B, Hv, -1), b=host(b), a=host(a)), host(y), \
        host(out)


@pytest.mark.parametrize("B,shape,P,pad", [
    (16, wl.RANK_LOCAL, 64, [3]),
    (256, wl.FULL_HEADS, 320, [0, 255]),
])
def test_decode_block(B, shape, P, pad):
    work = wl.decode_block(seed=B, B=B, P=P, s=shape)
    s, d = work.shape, work.data
    print(f"[block] {work.name} pad={pad}", flush=True)
    slots = d["slot_idx"].copy()
    slots[pad] = -1
    L = Layer(s, d["weights"])
    Pl = Pool(s, d["rec"], d["conv"])
    proj = oracle.Projections(**d["proj"])
    proj_d = {k: dev(v, torch.bfloat16) for k, v in d["proj"].items()}
    H = d["hidden"].shape[1]
    inp, y, out = _block_gpu(L, Pl, proj_d, slots, d["hidden"], s, H)
    rec_gpu, conv_gpu = host(Pl.rec), host(Pl.conv)

    # 1. the whole block against the oracle with no rounding between steps
    S_o, W_o = d["rec"].astype(np.float64), d["conv"].astype(np.float64)
    out_o, inp_o, _ = oracle.decode_block(L.og, L.ow, proj, S_o, W_o, slots, d["hidden"])
    assert_close("block out", maxrel_rows(out, out_o), TOL_BF16)
    for k in ("x", "b", "a"):
        assert_close(f"projection {k}", maxrel_rows(inp[k], inp_o[k]), TOL_BF16)
    assert_close("projection z", maxrel_rows(inp["z"].reshape(B, -1),
                                             inp_o["z"].reshape(B, -1)), TOL_BF16)

    # 2. the layer against the oracle fed the GPU's own bf16 projections
    S_g, W_g = d["rec"].astype(np.float64), d["conv"].astype(np.float64)
    y_g, _ = oracle.pool_run(L.og, L.ow, S_g, W_g, np.arange(B + 1), slots, inp["x"],
                             inp["z"], inp["a"], inp["b"])
    live = slots[slots >= 0]
    assert_close("y", maxrel_heads(y[slots >= 0], y_g[slots >= 0]), TOL_BF16)
    assert not y[slots < 0].any() and not out[slots < 0].any()
    assert_close("state", maxrel_states(rec_gpu[live], S_g[live]), TOL_F32)
    np.testing.assert_array_equal(conv_gpu[live], W_g[live])
    untouched = np.setdiff1d(np.arange(P), live)
    np.testing.assert_array_equal(rec_gpu[untouched], d["rec"][untouched])
