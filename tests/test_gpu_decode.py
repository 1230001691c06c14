"""GPU parity of batched decode (gdn_conv_update + gdn_decode_batch) against
the f64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_helpers import (TOL_F32, Layer, Pool, assert_close, decode_step, fused_step, host,
                         maxrel_heads, maxrel_states, y_tol)

pytestmark = pytest.mark.gpu


def _oracle_decode(L, rec, conv, slots, d):
    S = rec.astype(np.float64)
    W = conv.astype(np.float64)
    B = len(slots)
    y, o = oracle.pool_run(L.og, L.ow, S, W, np.arange(B + 1), slots, d["x"], d["z"],
                           d["a"], d["b"])
    return y, o, S, W


def _check_decode(work, rows=None):
    s, d = work.shape, work.data
    print(f"[decode] {work.name} seed={work.seed}", flush=True)
    L = Layer(s, d["weights"])
    P = Pool(s, d["rec"], d["conv"])
    slots = d["slot_idx"]
    y, o = decode_step(L, P, slots, d["x"], d["z"], d["a"], d["b"])
    torch.cuda.synchronize()
    rows = np.arange(len(slots)) if rows is None else np.asarray(rows)
    sub = {k: d[k][rows] for k in ("x", "z", "a", "b")}
    yo, oo, S, W = _oracle_decode(L, d["rec"], d["conv"], slots[rows], sub)
    assert_close("y", maxrel_heads(host(y)[rows], yo), y_tol(s))
    assert_close("o_raw", maxrel_heads(host(o)[rows], oo), TOL_F32)
    rec_gpu = host(P.rec)
    conv_gpu = host(P.conv)
    live = slots[rows]
    assert_close("state", maxrel_states(rec_gpu[live], S[live]), TOL_F32)
    np.testing.assert_array_equal(conv_gpu[live], W[live])   # raw inputs: exact
    untouched = np.setdiff1d(np.arange(d["rec"].shape[0]), slots)
    np.testing.assert_array_equal(rec_gpu[untouched], d["rec"][untouched])
    np.testing.assert_array_equal(conv_gpu[untouched], d["conv"][untouched])
    return L, P, y, o


def test_decode_tiny_f32():
    _check_decode(wl.decode_batch(seed=1, B=3, P=5, s=wl.TINY))


def test_decode_rank_local_b16():
    """16 rows, Hk=8, Hv=16, d=128, bf16 activations, 64-slot pool."""
    _check_decode(wl.decode_batch(seed=0))


def test_decode_slow_decay():
    _check_decode(wl.decode_batch(seed=3, B=8, P=12, slow_decay=True))


@pytest.mark.parametrize("d", [32, 64])
def test_decode_other_head_dims(d):
    s = wl.Shape(4, 8, d, d, 3, "bf16")
    _check_decode(wl.decode_batch(seed=4, B=5, P=9, s=s))


def test_decode_serving_shape_all_rows():
    """B=256 rows of a 320-slot pool at Hk=16, Hv=32, d=128: every row checked
    against the oracle (y, o_raw, states, windows), every untouched slot
    checked bit for bit."""
    _check_decode(wl.decode_batch(seed=5, B=256, P=320, s=wl.FULL_HEADS))


def test_decode_padding_rows():
    work = wl.decode_batch(seed=6, B=6, P=10)
    d = work.data
    slots = d["slot_idx"].copy()
    slots[[1, 4]] = -1
    L = Layer(work.shape, d["weights"])
    P = Pool(work.shape, d["rec"], d["conv"])
    y, o = decode_step(L, P, slots, d["x"], d["z"], d["a"], d["b"])
    yh, oh = host(y), host(o)
    assert not yh[[1, 4]].any() and not oh[[1, 4]].any()
    keep = np.array([0, 2, 3, 5])
    yo, oo, S, W = _oracle_decode(L, d["rec"], d["conv"], slots[keep],
                                  {k: d[k][keep] for k in ("x", "z", "a", "b")})
    assert_close("y", maxrel_heads(yh[keep], yo), y_tol(work.shape))
    rec = host(P.rec)
    untouched = np.setdiff1d(np.arange(10), slots[keep])
    np.testing.assert_array_equal(rec[untouched], d["rec"][untouched])


def test_decode_no_decay_no_write_keeps_state_bitwise():
    """A_log = -inf, b = -inf: g = 0 and beta = 0, so the state is unchanged
    bit for bit and o = S^T q."""
    work = wl.decode_batch(seed=7, B=4, P=6)
    d = work.data
    d["weights"]["A_log"][:] = -np.inf
    d["b"][:] = -np.inf
    L, P, y, o = _check_decode(work)
    np.testing.assert_array_equal(host(P.rec), d["rec"])


def test_decode_full_write_stores_value():
    """b = +inf gives beta = 1; with a unit key the updated state returns the
    value exactly: S'^T k_hat = v (checked on the GPU's own k and v)."""
    work = wl.decode_batch(seed=8, B=4, P=6, s=wl.TINY)
    d = work.data
    d["b"][:] = np.inf
    s = work.shape
    L = Layer(s, d["weights"])
    P = Pool(s, d["rec"], d["conv"])
    import linear_attention_causal_amd as gdn
    from gpu_helpers import dev
    slots = d["slot_idx"]
    sl = dev(slots, torch.int32)
    qkv = torch.empty(len(slots), s.channels, device="cuda")
    gdn.gdn_conv_update(L.geom, L.w, P.pool, sl, dev(d["x"]), qkv)
    y = torch.empty(len(slots), s.num_v_heads, s.head_v_dim, device="cuda")
    gdn.gdn_decode_batch(L.geom, L.w, P.pool, sl, qkv, dev(d["z"]), dev(d["a"]), dev(d["b"]), y)
    q = host(qkv)
    rec = host(P.rec)
    dk, Hk = s.head_k_dim, s.num_k_heads
    r = s.num_v_heads // Hk
    for row, slot in enumerate(slots):
        for h in range(s.num_v_heads):
            m = h // r
            k = q[row, Hk * dk + m * dk: Hk * dk + (m + 1) * dk].astype(np.float64)
            k /= np.sqrt((k * k).sum() + 1e-6)
            v = q[row, 2 * Hk * dk + h * s.head_v_dim: 2 * Hk * dk + (h + 1) * s.head_v_dim]
            got = rec[slot, h].T.astype(np.float64) @ k
            assert np.abs(got - v).max() <= 1e-4 * max(1.0, np.abs(v).max())


def test_decode_repeated_steps_match_oracle():
    """Eight consecutive decode steps on the same rows (state carried in the
    pool between launches)."""
    s = wl.Shape(4, 8, 64, 64, 4, "bf16")
    rng = np.random.default_rng(9)
    w = wl.layer_weights(rng, s)
    rec, conv = wl.state_pool(rng, s, 7)
    slots = np.array([5, 0, 3], np.int32)
    L = Layer(s, w)
    P = Pool(s, rec, conv)
    S, W = rec.astype(np.float64), conv.astype(np.float64)
    for step in range(8):
        inp = wl.token_inputs(rng, s, 3)
        y, o = decode_step(L, P, slots, inp["x"], inp["z"], inp["a"], inp["b"])
        yo, oo = oracle.pool_run(L.og, L.ow, S, W, np.arange(4), slots, inp["x"], inp["z"],
                                 inp["a"], inp["b"])
        assert_close(f"y step {step}", maxrel_heads(host(y), yo), y_tol(s))
    assert_close("state", maxrel_states(host(P.rec)[slots], S[slots]), TOL_F32)


# (shape, rows, pool slots): GQA ratios 1..4, head dims 32..128, conv
# widths 2..4, f32 and bf16 activations, a few rows to a few hundred.
@pytest.mark.parametrize("s,B,P", [(wl.TINY, 3, 5), (wl.RANK_LOCAL, 16, 64),
                                   (wl.RANK_LOCAL, 40, 64), (wl.RANK_LOCAL, 64, 80),
                                   (wl.FULL_HEADS, 64, 80), (wl.FULL_HEADS, 20, 30),
                                   (wl.Shape(4, 16, 64, 64, 3, "bf16"), 5, 9),
                                   (wl.Shape(4, 16, 64, 64, 3, "bf16"), 40, 50),
                                   (wl.Shape(4, 4, 64, 64, 2, "bf16"), 6, 8),
                                   (wl.Shape(2, 6, 32, 32, 4, "f32"), 4, 7),
                                   (wl.Shape(2, 6, 32, 32, 4, "f32"), 180, 200),
                                   (wl.Shape(2, 4, 64, 64, 4, "f32"), 9, 12),
                                   (wl.Shape(2, 4, 128, 128, 3, "f32"), 9, 12)])
def test_fused_decode_step_matches_oracle_and_two_calls(s, B, P):
    """gdn_decode_step (conv + state step + gated norm in one launch) against
    the oracle, and against gdn_conv_update + gdn_decode_batch on a copy of
    the same pools; a padding row included."""
    work = wl.decode_batch(seed=12, B=B, P=P, s=s)
    d = work.data
    slots = d["slot_idx"].copy()
    slots[B // 2] = -1
    L = Layer(s, d["weights"])
    P1, P2 = Pool(s, d["rec"], d["conv"]), Pool(s, d["rec"], d["conv"])
    print(f"[decode] fused step {work.name}", flush=True)
    y1, o1 = fused_step(L, P1, slots, d["x"], d["z"], d["a"], d["b"])
    y2, o2 = decode_step(L, P2, slots, d["x"], d["z"], d["a"], d["b"])
    torch.cuda.synchronize()
    assert not host(y1)[B // 2].any()
    np.testing.assert_allclose(host(o1), host(o2), rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(host(P1.rec), host(P2.rec), rtol=1e-5, atol=1e-6)
    np.testing.assert_array_equal(host(P1.conv), host(P2.conv))
    keep = np.array([i for i in range(B) if slots[i] >= 0])
    yo, oo, S, W = _oracle_decode(L, d["rec"], d["conv"], slots[keep],
                                  {k: d[k][keep] for k in ("x", "z", "a", "b")})
    assert_close("y", maxrel_heads(host(y1)[keep], yo), y_tol(s))
    assert_close("o_raw", maxrel_heads(host(o1)[keep], oo), TOL_F32)
    assert_close("state", maxrel_states(host(P1.rec)[slots[keep]], S[slots[keep]]), TOL_F32)
    np.testing.assert_array_equal(host(P1.conv)[slots[keep]], W[slots[keep]])
    untouched = np.setdiff1d(np.arange(P), slots[keep])
    np.testing.assert_array_equal(host(P1.rec)[untouched], d["rec"][untouched])


@pytest.mark.parametrize("s,sizes", [(wl.TINY, (6, 6, 200, 6, 150, 3)),
                                     (wl.Shape(4, 16, 64, 64, 3, "bf16"), (6, 40, 64, 6, 33, 70)),
                                     (wl.RANK_LOCAL, (6, 40, 70, 16, 63, 64))])
def test_fused_decode_steps_in_a_row_match_oracle(s, sizes):
    """Six gdn_decode_step calls in a row on one workspace (sized for the
    largest call) with changing row counts, rows moving between slots and one
    padding row, against the oracle's token loop.  The K-heads' q/k windows
    are written by the last of the workgroups that read them, which an
    arrival counter per (row, K-head) in the workspace decides; a counter left
    off zero by one call would leave a later call's windows unwritten or
    written early.  The workspace is also checked to be zero after the calls."""
    import linear_attention_causal_amd as gdn
    P = max(sizes) + 10
    work = wl.decode_batch(seed=31, B=4, P=P, s=s)
    d = work.data
    print(f"[decode] fused steps in a row {work.name} rows {sizes}", flush=True)
    L = Layer(s, d["weights"])
    Pg = Pool(s, d["rec"], d["conv"])
    S = d["rec"].astype(np.float64)
    W = d["conv"].astype(np.float64)
    rng = np.random.default_rng(8)
    ws = gdn.decode_workspace(L.geom, max(sizes))      # one workspace for every call
    for step, B in enumerate(sizes):
        slots = rng.choice(P, B, replace=False).astype(np.int32)
        slots[step % B] = -1
        inp = wl.token_inputs(rng, s, B)
        y, _ = fused_step(L, Pg, slots, inp["x"], inp["z"], inp["a"], inp["b"], workspace=ws,
                          want_o=False)
        keep = slots >= 0
        yo, _ = oracle.pool_run(L.og, L.ow, S, W, np.arange(keep.sum() + 1), slots[keep],
                                *(inp[k][keep] for k in ("x", "z", "a", "b")))
        torch.cuda.synchronize()
        assert_close(f"y step {step} (B={B})", maxrel_heads(host(y)[keep], yo), y_tol(s))
        assert not host(y)[~keep].any()
        np.testing.assert_array_equal(host(Pg.conv), W, err_msg=f"conv pool after step {step}")
    assert_close("state", maxrel_states(host(Pg.rec), S), TOL_F32)
    assert not ws.any(), "workspace not zero after the calls"


def test_fused_decode_step_large_pool_full_heads():
    """A full-head pool of 1100 slots (2.3 GB of state): rows in slots past
    1024 sit more than 2^31 bytes into the pool, so every state and window
    offset must be 64-bit.  Checked against the oracle on a compact copy of
    the used slots; the other slots stay untouched."""
    import linear_attention_causal_amd as gdn
    from gpu_helpers import act_dtype, dev
    s = wl.FULL_HEADS
    P_big = 1100
    work = wl.decode_batch(seed=5, B=5, P=6, s=s)
    d = work.data
    print(f"[decode] large full-head pool, {P_big} slots", flush=True)
    L = Layer(s, d["weights"])
    ad = act_dtype(s)
    place = np.array([1099, 7, 1050, 1024, 3, 512], np.int32)   # small-pool slot i -> big slot
    rec = torch.zeros(P_big, s.num_v_heads, s.head_k_dim, s.head_v_dim, device="cuda")
    conv = torch.zeros(P_big, s.conv_kernel, s.channels, device="cuda", dtype=ad)
    for i, j in enumerate(place):
        rec[int(j)] = dev(d["rec"][i])
        conv[int(j)] = dev(d["conv"][i], ad)
    pool = gdn.StatePool(L.geom, rec, conv)
    slots = d["slot_idx"]
    big = place[slots]
    ws = gdn.decode_workspace(L.geom, 5)
    y = torch.empty(5, s.num_v_heads, s.head_v_dim, device="cuda", dtype=ad)
    o = torch.empty(5, s.num_v_heads, s.head_v_dim, device="cuda")
    gdn.gdn_decode_step(L.geom, L.w, pool, dev(big, torch.int32),
                        *(dev(d[k], ad) for k in ("x", "z", "a", "b")), y, ws, o_raw=o,
                        slot_idx_host=big)
    yo, oo, S, W = _oracle_decode(L, d["rec"], d["conv"], slots,
                                  {k: d[k] for k in ("x", "z", "a", "b")})
    torch.cuda.synchronize()
    assert_close("y", maxrel_heads(host(y), yo), y_tol(s))
    assert_close("o_raw", maxrel_heads(host(o), oo), TOL_F32)
    idx = torch.from_numpy(place).long().cuda()
    assert_close("state", maxrel_states(host(rec[idx]), S), TOL_F32)
    np.testing.assert_array_equal(host(conv[idx]), W)
    others = torch.ones(P_big, dtype=torch.bool, device="cuda")
    others[idx] = False
    assert not rec[others].any() and not conv[others].any()


def test_two_pools_on_two_streams_same_slot_numbers():
    """Two layers' pools stepped at the same time on two streams, naming the
    same slot numbers, each call with its own workspace: nothing is shared
    between the calls (the arrival counters live in the workspaces), so both
    match the oracle."""
    import linear_attention_causal_amd as gdn
    s = wl.RANK_LOCAL
    B, P = 16, 24
    works = [wl.decode_batch(seed=40 + i, B=B, P=P, s=s) for i in range(2)]
    slots = works[0].data["slot_idx"]
    print(f"[decode] two pools, two streams, slots {slots.tolist()}", flush=True)
    Ls = [Layer(s, w.data["weights"]) for w in works]
    Ps = [Pool(s, w.data["rec"], w.data["conv"]) for w in works]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    wss = [gdn.decode_workspace(Ls[0].geom, B) for _ in range(2)]
    torch.cuda.synchronize()
    outs = []
    for rep in range(3):          # several rounds, each pair launched together
        inps = [wl.token_inputs(np.random.default_rng(100 * rep + i), s, B) for i in range(2)]
        res = []
        for i in range(2):
            res.append(fused_step(Ls[i], Ps[i], slots, *(inps[i][k] for k in ("x", "z", "a", "b")),
                                  workspace=wss[i], with_host=False, stream=streams[i]))
        torch.cuda.synchronize()
        outs.append((inps, [host(y) for y, _ in res], [host(o) for _, o in res]))
    for i, w in enumerate(works):
        S = w.data["rec"].astype(np.float64)
        W = w.data["conv"].astype(np.float64)
        for rep, (inps, ys, os_) in enumerate(outs):
            inp = inps[i]
            yo, oo = oracle.pool_run(Ls[i].og, Ls[i].ow, S, W, np.arange(B + 1), slots, inp["x"],
                                     inp["z"], inp["a"], inp["b"])
            assert_close(f"pool {i} round {rep} y", maxrel_heads(ys[i], yo), y_tol(s))
            assert_close(f"pool {i} round {rep} o_raw", maxrel_heads(os_[i], oo), TOL_F32)
        assert_close(f"pool {i} states", maxrel_states(host(Ps[i].rec)[slots], S[slots]), TOL_F32)
        np.testing.assert_array_equal(host(Ps[i].conv), W)
        assert not wss[i].any()
