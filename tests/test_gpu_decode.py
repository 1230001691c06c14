"""GPU parity of batched decode (gdn_conv_update + gdn_decode_batch) against
the f64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_helpers import (TOL_F32, Layer, Pool, assert_close, decode_step, host,
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


def test_decode_serving_shape_sampled():
    """B=256 rows of a 320-slot pool at Hk=16, Hv=32; 24 sampled rows checked
    against the oracle, every untouched slot checked bit for bit."""
    _check_decode(wl.decode_batch(seed=5, B=256, P=320, s=wl.FULL_HEADS),
                  rows=np.random.default_rng(5).choice(256, 24, replace=False))


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


@pytest.mark.parametrize("s,B,P", [(wl.TINY, 3, 5), (wl.RANK_LOCAL, 16, 64),
                                   (wl.FULL_HEADS, 64, 80), (wl.Shape(4, 16, 64, 64, 3, "bf16"), 5, 9),
                                   (wl.Shape(4, 4, 64, 64, 2, "bf16"), 6, 8),
                                   (wl.Shape(2, 6, 32, 32, 4, "f32"), 4, 7)])
def test_fused_decode_step_matches_oracle_and_two_calls(s, B, P):
    """gdn_decode_step (conv + state step + gated norm in one launch) against
    the oracle, and against gdn_conv_update + gdn_decode_batch on a copy of
    the same pools; a padding row included."""
    import linear_attention_causal_amd as gdn
    from gpu_helpers import act_dtype, dev
    work = wl.decode_batch(seed=12, B=B, P=P, s=s)
    d = work.data
    slots = d["slot_idx"].copy()
    slots[B // 2] = -1
    L = Layer(s, d["weights"])
    P1, P2 = Pool(s, d["rec"], d["conv"]), Pool(s, d["rec"], d["conv"])
    ad = act_dtype(s)
    y1 = torch.empty(B, s.num_v_heads, s.head_v_dim, device="cuda", dtype=ad)
    o1 = torch.empty(B, s.num_v_heads, s.head_v_dim, device="cuda")
    gdn.gdn_decode_step(L.geom, L.w, P1.pool, dev(slots, torch.int32), dev(d["x"], ad),
                        dev(d["z"], ad), dev(d["a"], ad), dev(d["b"], ad), y1, o1,
                        slot_idx_host=slots)
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


@pytest.mark.parametrize("s", [wl.TINY, wl.Shape(4, 16, 64, 64, 3, "bf16"), wl.RANK_LOCAL])
def test_fused_decode_steps_in_a_row_match_oracle(s):
    """Six gdn_decode_step calls in a row, rows moving between slots and one
    padding row, against the oracle's token loop.  The K-heads' q/k windows are
    written by the last of the Hv/Hk workgroups that read them, which an
    arrival counter per (slot, K-head) decides; a counter left off zero by one
    call would leave a later call's windows unwritten or written early."""
    import linear_attention_causal_amd as gdn
    from gpu_helpers import act_dtype, dev
    B, P = 6, 10
    work = wl.decode_batch(seed=31, B=B, P=P, s=s)
    d = work.data
    print(f"[decode] fused steps in a row {work.name}", flush=True)
    L = Layer(s, d["weights"])
    Pg = Pool(s, d["rec"], d["conv"])
    S = d["rec"].astype(np.float64)
    W = d["conv"].astype(np.float64)
    rng = np.random.default_rng(8)
    ad = act_dtype(s)
    for step in range(6):
        slots = rng.choice(P, B, replace=False).astype(np.int32)
        slots[step % B] = -1
        inp = wl.token_inputs(rng, s, B)
        y = torch.empty(B, s.num_v_heads, s.head_v_dim, device="cuda", dtype=ad)
        gdn.gdn_decode_step(L.geom, L.w, Pg.pool, dev(slots, torch.int32),
                            *(dev(inp[k], ad) for k in ("x", "z", "a", "b")), y,
                            slot_idx_host=slots)
        keep = slots >= 0
        yo, _ = oracle.pool_run(L.og, L.ow, S, W, np.arange(keep.sum() + 1), slots[keep],
                                *(inp[k][keep] for k in ("x", "z", "a", "b")))
        torch.cuda.synchronize()
        assert_close(f"y step {step}", maxrel_heads(host(y)[keep], yo), y_tol(s))
        assert not host(y)[~keep].any()
        np.testing.assert_array_equal(host(Pg.conv), W, err_msg=f"conv pool after step {step}")
    assert_close("state", maxrel_states(host(Pg.rec), S), TOL_F32)


def test_fused_decode_step_large_pool_fallback():
    """A pool with more (slot, K-head) pairs than the arrival counters cover
    runs the per-K-head kernel; slots beyond that bound are read and written
    correctly (checked against the oracle on a compact copy of the used slots)."""
    import linear_attention_causal_amd as gdn
    from gpu_helpers import act_dtype, dev
    s = wl.TINY                      # Hk = 2, one wave of q/k channels per K-head
    P_big = 32769                    # 2 * 32769 counters needed: past the table
    work = wl.decode_batch(seed=5, B=3, P=4, s=s)
    d = work.data
    print(f"[decode] large pool fallback, {P_big} slots", flush=True)
    L = Layer(s, d["weights"])
    ad = act_dtype(s)
    place = np.array([32768, 7, 20000, 31], np.int32)     # small-pool slot i -> big slot
    rec = torch.zeros(P_big, s.num_v_heads, s.head_k_dim, s.head_v_dim, device="cuda")
    conv = torch.zeros(P_big, s.conv_kernel, s.channels, device="cuda", dtype=ad)
    for i, j in enumerate(place):
        rec[int(j)] = dev(d["rec"][i])
        conv[int(j)] = dev(d["conv"][i], ad)
    pool = gdn.StatePool(L.geom, rec, conv)
    slots = d["slot_idx"]
    big = place[slots]
    y = torch.empty(3, s.num_v_heads, s.head_v_dim, device="cuda", dtype=ad)
    gdn.gdn_decode_step(L.geom, L.w, pool, dev(big, torch.int32),
                        *(dev(d[k], ad) for k in ("x", "z", "a", "b")), y, slot_idx_host=big)
    yo, _, S, W = _oracle_decode(L, d["rec"], d["conv"], slots,
                                 {k: d[k] for k in ("x", "z", "a", "b")})
    torch.cuda.synchronize()
    assert_close("y", maxrel_heads(host(y), yo), y_tol(s))
    assert_close("state", maxrel_states(host(rec[torch.from_numpy(place).long()]), S), TOL_F32)
    np.testing.assert_array_equal(host(conv[torch.from_numpy(place).long()]), W)
