"""GPU parity of chunkwise prefill (gdn_prefill_chunked) against the f64
oracle, through the C ABI: ragged and packed sequences, the tiny f32 layer
(prefill then decode), the rank-local 4096-token prefill and the packed
varlen prefill at full head count."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_helpers import (TOL_F32, Layer, Pool, assert_close, decode_step, host,
                         maxrel_heads, maxrel_states, prefill, y_tol)

pytestmark = pytest.mark.gpu


def _oracle_prefill(L, rec, conv, cu, slots, d, has_init=None, heads=None):
    """Oracle of a packed prefill on a pool; with `heads` only those V-heads
    are computed (states of other heads are then not meaningful)."""
    S = rec.astype(np.float64)
    W = conv.astype(np.float64)
    if heads is None:
        y, o = oracle.pool_run(L.og, L.ow, S, W, cu, slots, d["x"], d["z"], d["a"], d["b"],
                               has_init=has_init)
        return y, o, S, W
    N = len(cu) - 1
    S0 = np.stack([S[s] if (has_init is None or has_init[n]) else np.zeros_like(S[0])
                   for n, s in enumerate(slots)])
    W0 = np.stack([W[s] if (has_init is None or has_init[n]) else np.zeros_like(W[0])
                   for n, s in enumerate(slots)])
    mask = np.zeros(L.s.num_v_heads, np.uint8)
    mask[list(heads)] = 1
    y, o, Sn, Wn = oracle.sequences(L.og, L.ow, cu, d["x"], d["z"], d["a"], d["b"], S0, W0,
                                    head_mask=mask)
    for n, s in enumerate(slots):
        S[s] = Sn[n]
        W[s] = Wn[n]
    return y, o, S, W


def _check_prefill(s, w, rec, conv, cu, slots, d, has_init=None, heads=None, tag="",
                   want_o=True):
    """Parity of one packed prefill; want_o=False makes the call without o_raw
    (a bf16 layer then takes its bf16 output path) and checks y and the states."""
    print(f"[prefill] {tag} T={int(cu[-1])} N={len(cu) - 1} o_raw={want_o}", flush=True)
    L = Layer(s, w)
    P = Pool(s, rec, conv)
    y, o = prefill(L, P, cu, slots, d["x"], d["z"], d["a"], d["b"], has_init=has_init,
                   want_o=want_o)
    torch.cuda.synchronize()
    yo, oo, S, W = _oracle_prefill(L, rec, conv, cu, slots, d, has_init, heads)
    hs = np.arange(s.num_v_heads) if heads is None else np.asarray(heads)
    yh = host(y)
    oh = host(o) if want_o else np.zeros_like(yh)
    live = np.asarray([sl for sl in slots if sl >= 0])
    tok = np.concatenate([np.arange(cu[n], cu[n + 1]) for n in range(len(slots))
                          if slots[n] >= 0] + [np.zeros(0, np.int64)]).astype(np.int64)
    if tok.size:
        assert_close("y", maxrel_heads(yh[tok][:, hs], yo[tok][:, hs]), y_tol(s))
        if want_o:
            assert_close("o_raw", maxrel_heads(oh[tok][:, hs], oo[tok][:, hs]), TOL_F32)
    rec_gpu, conv_gpu = host(P.rec), host(P.conv)
    if live.size:
        assert_close("state", maxrel_states(rec_gpu[live][:, hs], S[live][:, hs]), TOL_F32)
        np.testing.assert_array_equal(conv_gpu[live], W[live])
    pad_tok = np.concatenate([np.arange(cu[n], cu[n + 1]) for n in range(len(slots))
                              if slots[n] < 0] + [np.zeros(0, np.int64)]).astype(np.int64)
    assert not yh[pad_tok].any() and not oh[pad_tok].any()
    untouched = np.setdiff1d(np.arange(rec.shape[0]), live)
    np.testing.assert_array_equal(rec_gpu[untouched], rec[untouched])
    np.testing.assert_array_equal(conv_gpu[untouched], conv[untouched])
    return L, P, y, o


def _packed(seed, s, lens, P, slow=False):
    rng = np.random.default_rng(seed)
    w = wl.layer_weights(rng, s, slow)
    rec, conv = wl.state_pool(rng, s, P)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    d = wl.token_inputs(rng, s, int(cu[-1]))
    return w, rec, conv, cu, d


@pytest.mark.parametrize("T", [1, 2, 5, 63, 64, 65, 130, 200])
def test_prefill_ragged_single(T):
    s = wl.Shape(2, 4, 32, 32, 4, "f32")
    w, rec, conv, cu, d = _packed(100 + T, s, [T], 2)
    _check_prefill(s, w, rec, conv, cu, np.array([1], np.int32), d, tag=f"f32 d32 T={T}")


@pytest.mark.parametrize("D,K", [(64, 4), (128, 3)])
def test_prefill_packed_f32_wide_heads(D, K):
    """f32 activations at head dims 64 and 128 (16-byte runs of four
    channels in the conv tiles): packed sequences with partial chunks, a
    one-token sequence, a fresh start and a padding sequence."""
    s = wl.Shape(2, 4, D, D, K, "f32")
    lens = [70, 130, 1, 64, 17]
    slots = np.array([3, 0, 5, -1, 1], np.int32)
    init = np.array([1, 1, 1, 1, 0], np.uint8)
    w, rec, conv, cu, d = _packed(400 + D + K, s, lens, 7)
    _check_prefill(s, w, rec, conv, cu, slots, d, has_init=init, tag=f"packed f32 d{D} K={K}")


@pytest.mark.parametrize("want_o", [True, False])
def test_prefill_packed_mixed_bf16(want_o):
    """Packed sequences with a zero-length one, a fresh start (has_init = 0),
    a padding sequence (slot -1) and partial last chunks."""
    s = wl.Shape(4, 8, 64, 64, 4, "bf16")
    lens = [70, 0, 3, 129, 64, 17]
    slots = np.array([4, 0, 7, -1, 2, 5], np.int32)
    init = np.array([1, 1, 0, 1, 0, 1], np.uint8)
    w, rec, conv, cu, d = _packed(200, s, lens, 9)
    _check_prefill(s, w, rec, conv, cu, slots, d, has_init=init, tag="packed bf16 d64",
                   want_o=want_o)


@pytest.mark.parametrize("K", [2, 3])
def test_prefill_conv_widths(K):
    s = wl.Shape(2, 4, 32, 32, K, "bf16")
    w, rec, conv, cu, d = _packed(300 + K, s, [2, 90], 3)
    _check_prefill(s, w, rec, conv, cu, np.array([2, 0], np.int32), d, tag=f"K={K}")


@pytest.mark.parametrize("want_o", [True, False])
def test_prefill_many_sequences_device_prefix(want_o):
    """70 packed sequences (more than the launch carries inline, so the chunk
    prefix is formed on the device), with empty ones, padding and fresh starts."""
    s = wl.Shape(2, 4, 32, 32, 4, "bf16")
    rng = np.random.default_rng(600)
    N, P = 70, 80
    lens = rng.integers(0, 90, N)
    lens[[3, 17, 40]] = 0
    slots = rng.choice(P, N, replace=False).astype(np.int32)
    slots[[5, 33]] = -1
    init = (rng.random(N) < 0.7).astype(np.uint8)
    w, rec, conv, cu, d = _packed(601, s, list(lens), P)
    _check_prefill(s, w, rec, conv, cu, slots, d, has_init=init, tag="70 sequences",
                   want_o=want_o)


@pytest.mark.parametrize("want_o", [True, False])
@pytest.mark.parametrize("N", [3, 70])
def test_prefill_all_sequences_empty(N, want_o):
    """No tokens at all (T = 0, no scratch): each slot keeps its state and
    window, or is reset to zeros for a fresh start; padding untouched."""
    s = wl.Shape(2, 4, 32, 32, 4, "bf16")
    rng = np.random.default_rng(700 + N)
    P = N + 5
    slots = rng.choice(P, N, replace=False).astype(np.int32)
    slots[1] = -1
    init = (rng.random(N) < 0.5).astype(np.uint8)
    w, rec, conv, cu, d = _packed(701 + N, s, [0] * N, P)
    _check_prefill(s, w, rec, conv, cu, slots, d, has_init=init, tag=f"{N} empty sequences",
                   want_o=want_o)


@pytest.mark.parametrize("want_o", [True, False])
@pytest.mark.parametrize("Hk,Hv", [(1, 8), (2, 6), (4, 4)])
def test_prefill_gqa_ratios(Hk, Hv, want_o):
    """8, 3 and 1 V-heads per K-head (the prep kernel forms the gates in
    groups of up to four V-heads)."""
    s = wl.Shape(Hk, Hv, 32, 32, 4, "bf16")
    w, rec, conv, cu, d = _packed(500 + Hv, s, [97, 40], 3)
    _check_prefill(s, w, rec, conv, cu, np.array([2, 0], np.int32), d, tag=f"Hk={Hk} Hv={Hv}",
                   want_o=want_o)


def test_prefill_slow_decay_long_carry():
    """Slow decay (e^g ~ 0.98..0.998) so the state carries across many chunks."""
    s = wl.RANK_LOCAL
    w, rec, conv, cu, d = _packed(400, s, [700], 1, slow=True)
    _check_prefill(s, w, rec, conv, cu, np.array([0], np.int32), d, tag="slow decay d128")


def test_tiny_prefill_then_decode_f32():
    """Tiny f32 layer: a 64-token prefill then 8 decode steps, against the
    oracle, and against one 72-token prefill on the GPU."""
    work = wl.tiny(seed=0)
    s, d = work.shape, work.data
    L = Layer(s, d["weights"])
    P = Pool(s, d["rec"], d["conv"])
    pre = d["prefill"]
    y, o = prefill(L, P, d["cu_seqlens"], d["slot_idx"], pre["x"], pre["z"], pre["a"], pre["b"])
    S, W = d["rec"].astype(np.float64), d["conv"].astype(np.float64)
    yo, oo = oracle.pool_run(L.og, L.ow, S, W, d["cu_seqlens"], d["slot_idx"], pre["x"],
                             pre["z"], pre["a"], pre["b"])
    assert_close("prefill y", maxrel_heads(host(y), yo), TOL_F32)
    assert_close("prefill o", maxrel_heads(host(o), oo), TOL_F32)
    ys = [host(y)]
    for step in d["steps"]:
        yd, od = decode_step(L, P, d["slot_idx"], step["x"], step["z"], step["a"], step["b"])
        yo, oo = oracle.pool_run(L.og, L.ow, S, W, [0, 1], d["slot_idx"], step["x"], step["z"],
                                 step["a"], step["b"])
        assert_close("decode y", maxrel_heads(host(yd), yo), TOL_F32)
        ys.append(host(yd))
    assert_close("state", maxrel_states(host(P.rec), S), TOL_F32)
    np.testing.assert_array_equal(host(P.conv), W)
    # the same 72 tokens as one prefill on a fresh pool
    cat = {k: np.concatenate([pre[k]] + [st[k] for st in d["steps"]]) for k in pre}
    P2 = Pool(s, d["rec"], d["conv"])
    y72, _ = prefill(L, P2, [0, 72], [0], cat["x"], cat["z"], cat["a"], cat["b"])
    assert_close("prefill(72) vs prefill(64)+8 decode",
                 maxrel_heads(host(y72), np.concatenate(ys)), TOL_F32)
    assert_close("state handoff", maxrel_states(host(P2.rec), host(P.rec)), TOL_F32)


def test_prefill_rank_local_t4096():
    """One 4096-token sequence, Hk=8, Hv=16, d=128, bf16, N(0, 0.1) initial
    state; every head checked."""
    work = wl.prefill_single(seed=0)
    d = work.data
    _check_prefill(work.shape, d["weights"], d["rec"], d["conv"], d["cu_seqlens"],
                   d["slot_idx"], d, has_init=d["has_init"], tag=work.name)


def test_prefill_varlen8_full_heads():
    """Eight packed sequences of U(128, 8192) tokens at Hk=16, Hv=32, d=128,
    per-sequence nonzero initial states, with o_raw: every V-head's y, o_raw
    and final state, every conv window, against the oracle."""
    work = wl.prefill_varlen(seed=0)
    d = work.data
    _check_prefill(work.shape, d["weights"], d["rec"], d["conv"], d["cu_seqlens"],
                   d["slot_idx"], d, has_init=d["has_init"], tag=work.name)


@pytest.mark.parametrize("lens,P", [([70, 1, 200, 64, 129], 8), ([300, 17, 64, 5, 130, 90, 1], 9)])
def test_prefill_32_column_state_tiles_with_o_raw(lens, P):
    """d=128 with o_raw at batch sizes whose state workgroups take 32 of the
    128 state columns (5 or 7 sequences x 16 V-heads: the widest tile that
    still gives about one workgroup per CU), including partial and one-token
    chunks and a fresh start."""
    s = wl.RANK_LOCAL
    w, rec, conv, cu, d = _packed(800 + len(lens), s, lens, P)
    slots = np.random.default_rng(len(lens)).choice(P, len(lens), replace=False).astype(np.int32)
    init = np.ones(len(lens), np.uint8)
    init[1] = 0
    _check_prefill(s, w, rec, conv, cu, slots, d, has_init=init, tag=f"32-column tiles {lens}")


def test_prefill_equals_decode_steps():
    """Property at any size: a prefill of T tokens equals T decode steps."""
    s = wl.RANK_LOCAL
    w, rec, conv, cu, d = _packed(500, s, [150], 2)
    L = Layer(s, w)
    Pa = Pool(s, rec, conv)
    ya, _ = prefill(L, Pa, cu, [1], d["x"], d["z"], d["a"], d["b"])
    Pb = Pool(s, rec, conv)
    ys = []
    for t in range(150):
        yt, _ = decode_step(L, Pb, [1], d["x"][t:t + 1], d["z"][t:t + 1], d["a"][t:t + 1],
                            d["b"][t:t + 1], want_o=False)
        ys.append(host(yt))
    assert_close("y", maxrel_heads(host(ya), np.concatenate(ys)), y_tol(s))
    assert_close("state", maxrel_states(host(Pa.rec)[1], host(Pb.rec)[1]), TOL_F32)
    np.testing.assert_array_equal(host(Pa.conv), host(Pb.conv))


@pytest.mark.parametrize("case", ["packed", "narrow", "t4096", "varlen"])
def test_prefill_without_o_raw(case):
    """The call without o_raw, as a serving caller makes it (the pre-norm
    output then stays internal): y, states and conv windows against the
    oracle, padding rows zero, untouched slots unchanged.  "narrow" has few
    enough sequences for 16-column state tiles, with partial last chunks."""
    if case == "packed":
        s = wl.RANK_LOCAL
        w, rec, conv, cu, d = _packed(700, s, [70, 1, 200, 64, 129], 8)
        slots, has_init = [5, 0, -1, 2, 7], [1, 1, 1, 0, 1]
    elif case == "narrow":
        s = wl.RANK_LOCAL
        w, rec, conv, cu, d = _packed(701, s, [70, 5, 129], 8)
        slots, has_init = [3, -1, 6], [1, 1, 0]
    else:
        work = wl.prefill_single(seed=0) if case == "t4096" else wl.prefill_varlen(seed=0)
        s, d = work.shape, work.data
        w, rec, conv, cu = d["weights"], d["rec"], d["conv"], d["cu_seqlens"]
        slots, has_init = d["slot_idx"], d["has_init"]
    heads = None
    print(f"[prefill without o_raw] {case} T={int(cu[-1])}", flush=True)
    L = Layer(s, w)
    P = Pool(s, rec, conv)
    y, _ = prefill(L, P, cu, slots, d["x"], d["z"], d["a"], d["b"], has_init=has_init,
                   want_o=False)
    torch.cuda.synchronize()
    yo, _, S, W = _oracle_prefill(L, rec, conv, cu, slots, d, np.asarray(has_init, np.uint8),
                                  heads=heads)
    hs = np.arange(s.num_v_heads) if heads is None else np.asarray(heads)
    yh = host(y)
    live = np.asarray([sl for sl in slots if sl >= 0])
    tok = np.concatenate([np.arange(cu[n], cu[n + 1]) for n in range(len(slots))
                          if slots[n] >= 0]).astype(np.int64)
    assert_close("y", maxrel_heads(yh[tok][:, hs], yo[tok][:, hs]), y_tol(s))
    assert_close("state", maxrel_states(host(P.rec)[live][:, hs], S[live][:, hs]), TOL_F32)
    np.testing.assert_array_equal(host(P.conv)[live], W[live])
    pad = np.concatenate([np.arange(cu[n], cu[n + 1]) for n in range(len(slots))
                          if slots[n] < 0] + [np.zeros(0, np.int64)]).astype(np.int64)
    assert not yh[pad].any()
    untouched = np.setdiff1d(np.arange(rec.shape[0]), live)
    np.testing.assert_array_equal(host(P.rec)[untouched], rec[untouched])


@pytest.mark.parametrize("want_o", [True, False])
def test_prefill_imbalanced_packed_batch(want_o):
    """Eight packed sequences at Hk=8, Hv=16, d=128 (64-column state tiles)
    with one much longer than the rest, partial chunks, a one-token
    sequence, a fresh start and a padding sequence: every head of y (and
    o_raw), every state and window against the oracle."""
    s = wl.RANK_LOCAL
    lens = [1000, 64, 70, 5, 130, 64, 1, 200]
    w, rec, conv, cu, d = _packed(900, s, lens, 12)
    slots = np.array([3, 0, 7, 11, -1, 5, 9, 2], np.int32)
    init = np.array([1, 1, 0, 1, 1, 1, 1, 1], np.uint8)
    _check_prefill(s, w, rec, conv, cu, slots, d, has_init=init, tag="imbalanced packed batch",
                   want_o=want_o)


@pytest.mark.parametrize("want_o", [True, False])
def test_prefill_sequence_order_invariance(want_o):
    """Each sequence of a packed batch is computed on its own (its chunks
    never span another's, and the state pass takes the sequences longest
    first whatever their order): the same sequences packed in reverse order,
    with their slots and flags, give bit-identical y (and o_raw), states and
    conv windows.  64-column state tiles (Hk=8, Hv=16, d=128, eight
    sequences)."""
    s = wl.RANK_LOCAL
    lens = [1000, 64, 70, 5, 130, 64, 1, 200]
    w, rec, conv, cu, d = _packed(950, s, lens, 12)
    slots = np.array([3, 0, 7, 11, -1, 5, 9, 2], np.int32)
    init = np.array([1, 1, 0, 1, 1, 1, 1, 1], np.uint8)
    L = Layer(s, w)
    rev = np.arange(len(lens))[::-1]
    lens_r = [lens[n] for n in rev]
    cu_r = np.concatenate([[0], np.cumsum(lens_r)]).astype(np.int32)
    tok_r = np.concatenate([np.arange(cu[n], cu[n + 1]) for n in rev]).astype(np.int64)
    d_r = {k: d[k][tok_r] for k in ("x", "z", "a", "b")}
    runs = []
    for order, (c, sl, hi, dd) in enumerate(((cu, slots, init, d), (cu_r, slots[rev], init[rev], d_r))):
        print(f"[prefill] order invariance, packing {order} o_raw={want_o}", flush=True)
        P = Pool(s, rec, conv)
        y, o = prefill(L, P, c, sl, dd["x"], dd["z"], dd["a"], dd["b"], has_init=hi,
                       want_o=want_o)
        torch.cuda.synchronize()
        runs.append((host(y), host(o) if want_o else None, host(P.rec), host(P.conv)))
    (y0, o0, r0, c0), (y1, o1, r1, c1) = runs
    # row t of the reversed packing holds row tok_r[t] of the original one
    np.testing.assert_array_equal(y1, y0[tok_r])
    if want_o:
        np.testing.assert_array_equal(o1, o0[tok_r])
    np.testing.assert_array_equal(r1, r0)
    np.testing.assert_array_equal(c1, c0)
