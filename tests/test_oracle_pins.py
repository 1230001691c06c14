"""Pins of the double-precision oracle against facts that do not come from the
oracle itself: library routines (torch conv1d / rms_norm in f64), closed
forms, invariants of the gated delta rule, an independent numpy
transition-matrix form on tiny shapes, and special cases that reduce to a
plain matmul.  CPU only."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import bruteforce
from workloads import Shape, layer_weights, token_inputs

G = oracle.Geometry(2, 4, 8, 6, 4)


def _rand_layer(rng, geom, T, init=True):
    C, K = geom.channels, geom.conv_kernel
    Hv, dk, dv = geom.num_v_heads, geom.head_k_dim, geom.head_v_dim
    w = oracle.Weights(rng.normal(0, 0.5, (C, K)), np.log(rng.uniform(0.05, 3, Hv)),
                       rng.uniform(-1, 1, Hv), 1 + 0.1 * rng.normal(size=dv))
    x = rng.normal(size=(T, C))
    z = rng.normal(size=(T, Hv, dv))
    a = rng.normal(size=(T, Hv))
    b = rng.normal(size=(T, Hv))
    S0 = rng.normal(0, 0.3, (Hv, dk, dv)) if init else np.zeros((Hv, dk, dv))
    W0 = rng.normal(size=(K, C)) if init else np.zeros((K, C))
    return w, x, z, a, b, S0, W0


def _run(geom, w, x, z, a, b, S0, W0, chunk=0):
    T = x.shape[0]
    y, o, S, W = oracle.sequences(geom, w, [0, T], x, z, a, b, S0[None], W0[None],
                                  chunk=chunk)
    return y, o, S[0], W[0]


# ------------------------------------------------------------------ conv


def test_conv_matches_torch_conv1d_zero_window():
    rng = np.random.default_rng(1)
    T, C, K = 11, 5, 4
    w, x = rng.normal(size=(C, K)), rng.normal(size=(T, C))
    got = oracle.conv_silu(w, np.zeros((K, C)), x)
    xt = torch.from_numpy(x.T[None].copy())
    ref = torch.nn.functional.conv1d(xt, torch.from_numpy(w[:, None, :].copy()),
                                     groups=C, padding=K - 1)[0, :, :T].T
    ref = torch.nn.functional.silu(ref).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-13)


def test_conv_matches_torch_conv1d_with_window():
    rng = np.random.default_rng(2)
    T, C, K = 6, 7, 3
    w, x, win = rng.normal(size=(C, K)), rng.normal(size=(T, C)), rng.normal(size=(K, C))
    got = oracle.conv_silu(w, win, x)
    # the window's newest K-1 columns precede the first token
    stream = np.concatenate([win[1:], x])
    ref = torch.nn.functional.conv1d(torch.from_numpy(stream.T[None].copy()),
                                     torch.from_numpy(w[:, None, :].copy()), groups=C)
    ref = torch.nn.functional.silu(ref[0].T).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-13)


def test_conv_identity_tap_is_silu():
    rng = np.random.default_rng(3)
    T, C, K = 9, 4, 4
    w = np.zeros((C, K))
    w[:, K - 1] = 1.0
    x = rng.normal(size=(T, C))
    got = oracle.conv_silu(w, rng.normal(size=(K, C)), x)
    # numpy's exp and libm's may differ in the last bit
    np.testing.assert_allclose(got, x / (1 + np.exp(-x)), rtol=1e-15, atol=0)


@pytest.mark.parametrize("T", [1, 2, 3, 4, 9])
def test_conv_window_is_last_k_inputs(T):
    rng = np.random.default_rng(4)
    w, x, z, a, b, S0, W0 = _rand_layer(rng, G, T)
    _, _, _, W = _run(G, w, x, z, a, b, S0, W0)
    np.testing.assert_array_equal(W, np.concatenate([W0, x])[-G.conv_kernel:])


# ------------------------------------------------------------ l2norm, gates


def test_l2norm_unit_and_scaled():
    rng = np.random.default_rng(5)
    x = rng.normal(size=128)
    assert abs(np.linalg.norm(oracle.l2norm(x, 1e-6)) - 1) < 1e-7
    assert abs(np.linalg.norm(oracle.l2norm(x, 0.0, 1 / math.sqrt(128))) - 128 ** -0.5) < 1e-15
    # eps enters under the square root: x / sqrt(|x|^2 + eps)
    e = oracle.l2norm(np.array([3.0, 4.0]), 11.0)
    np.testing.assert_allclose(e, [0.5, 4 / 6], rtol=1e-15)


def test_softplus_and_gate_closed_forms():
    assert oracle.softplus(0.0) == pytest.approx(math.log(2), rel=1e-15)
    assert oracle.softplus(50.0) == pytest.approx(50.0, rel=1e-15)
    assert oracle.softplus(-50.0) == pytest.approx(math.exp(-50), rel=1e-12)
    # a + dt_bias = 0  ->  g = -exp(A_log) ln 2 ; b = 0 -> beta = 1/2
    g, beta = oracle.gates(math.log(3.0), 0.25, -0.25, 0.0)
    assert g == pytest.approx(-3 * math.log(2), rel=1e-15)
    assert beta == 0.5
    g, beta = oracle.gates(math.log(2.0), 1.0, 0.5, 2.0)
    assert g == pytest.approx(-2 * math.log1p(math.exp(1.5)), rel=1e-15)
    assert beta == pytest.approx(1 / (1 + math.exp(-2)), rel=1e-15)
    # limits: no decay, full / no write
    g, beta = oracle.gates(-math.inf, 0.3, 0.7, math.inf)
    assert g == 0.0 and beta == 1.0
    _, beta = oracle.gates(0.0, 0.0, 0.0, -math.inf)
    assert beta == 0.0


# ------------------------------------------------------------ recurrence


def test_step_no_decay_no_write_keeps_state():
    rng = np.random.default_rng(6)
    S = rng.normal(size=(8, 6))
    q, k, v = rng.normal(size=8), oracle.l2norm(rng.normal(size=8)), rng.normal(size=6)
    S1, o = oracle.gdr_step(0.0, 0.0, k, v, q, S)
    np.testing.assert_array_equal(S1, S)
    np.testing.assert_allclose(o, S.T @ q, rtol=1e-14)


@pytest.mark.parametrize("g", [0.0, -0.3, -4.0])
def test_step_full_write_stores_value(g):
    """beta = 1 and a unit key: afterwards S^T k equals v whatever the decay."""
    rng = np.random.default_rng(7)
    S = rng.normal(size=(8, 6))
    k = rng.normal(size=8)
    k /= np.linalg.norm(k)
    v, q = rng.normal(size=6), rng.normal(size=8)
    S1, o = oracle.gdr_step(g, 1.0, k, v, q, S)
    np.testing.assert_allclose(S1.T @ k, v, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(o, S1.T @ q, rtol=1e-13)   # output reads S_t


def test_layer_no_decay_no_write_through_gates():
    """A_log = -inf and b = -inf make g = 0, beta = 0: the state is unchanged
    and o_t = S_0^T q_t."""
    rng = np.random.default_rng(8)
    w, x, z, a, b, S0, W0 = _rand_layer(rng, G, 10)
    w.A_log[:] = -np.inf
    b[:] = -np.inf
    y, o, S, _ = _run(G, w, x, z, a, b, S0, W0)
    np.testing.assert_array_equal(S, S0)
    _, _, Sb, _ = bruteforce.layer(G, w.conv_w, w.A_log, w.dt_bias, w.norm_w, x, z, a, b,
                                   S0, W0)
    np.testing.assert_allclose(S, Sb, atol=0)


def test_pure_decay():
    """beta = 0: S_T = e^{sum g} S_0 and o_t = e^{gamma_t} S_0^T q_t."""
    rng = np.random.default_rng(9)
    geom = oracle.Geometry(2, 4, 8, 6, 4, l2norm_eps=0.0)
    w, x, z, a, b, S0, W0 = _rand_layer(rng, geom, 7)
    b[:] = -np.inf
    y, o, S, _ = _run(geom, w, x, z, a, b, S0, W0)
    g = -np.exp(w.A_log) * np.logaddexp(0, a + w.dt_bias)          # [T][Hv]
    gam = np.cumsum(g, axis=0)
    np.testing.assert_allclose(S, np.exp(gam[-1])[:, None, None] * S0, rtol=1e-12)
    act = oracle.conv_silu(w.conv_w, W0, x)
    r = geom.num_v_heads // geom.num_k_heads
    for h in range(geom.num_v_heads):
        m = h // r
        for t in range(x.shape[0]):
            qh = oracle.l2norm(act[t, m * 8:(m + 1) * 8], 0.0, 8 ** -0.5)
            np.testing.assert_allclose(o[t, h], np.exp(gam[t, h]) * S0[h].T @ qh,
                                       rtol=1e-11, atol=1e-14)


def test_orthogonal_keys_reduce_to_masked_matmul():
    """Identity conv tap, one-hot keys (k_t = e_t), zero initial state: the
    delta correction vanishes and O = (M * Q K^T) diag(beta) V with
    M_ts = e^{gamma_t - gamma_s} for s <= t, else 0."""
    rng = np.random.default_rng(10)
    Hk, Hv, dk, dv, K = 1, 2, 8, 5, 4
    geom = oracle.Geometry(Hk, Hv, dk, dv, K, l2norm_eps=0.0)
    C, T = geom.channels, 8
    conv_w = np.zeros((C, K))
    conv_w[:, K - 1] = 1.0
    w = oracle.Weights(conv_w, np.log(rng.uniform(0.1, 2, Hv)), rng.uniform(-1, 1, Hv),
                       np.ones(dv))
    x = rng.normal(size=(T, C))
    x[:, dk:2 * dk] = 0.0
    for t in range(T):
        x[t, dk + t] = 1.5 + rng.uniform()         # SiLU > 0, the only nonzero key entry
    z, a, b = rng.normal(size=(T, Hv, dv)), rng.normal(size=(T, Hv)), rng.normal(size=(T, Hv))
    _, o, _, _ = _run(geom, w, x, z, a, b, np.zeros((Hv, dk, dv)), np.zeros((K, C)))
    silu = x / (1 + np.exp(-x))
    Q = np.stack([oracle.l2norm(silu[t, :dk], 0.0, dk ** -0.5) for t in range(T)])
    Kk = np.eye(dk)[:T]
    for h in range(Hv):
        g = -np.exp(w.A_log[h]) * np.logaddexp(0, a[:, h] + w.dt_bias[h])
        gam = np.cumsum(g)
        M = np.tril(np.exp(gam[:, None] - gam[None, :]))
        beta = 1 / (1 + np.exp(-b[:, h]))
        V = silu[:, 2 * dk + h * dv: 2 * dk + (h + 1) * dv]
        ref = (M * (Q @ Kk.T)) @ np.diag(beta) @ V
        np.testing.assert_allclose(o[:, h], ref, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("seed,T,init", [(11, 1, True), (12, 5, True), (13, 9, False),
                                         (14, 13, True)])
def test_matches_transition_matrix_bruteforce(seed, T, init):
    rng = np.random.default_rng(seed)
    geom = oracle.Geometry(2, 6, 5, 4, 3)
    w, x, z, a, b, S0, W0 = _rand_layer(rng, geom, T, init)
    y, o, S, W = _run(geom, w, x, z, a, b, S0, W0)
    yb, ob, Sb, Wb = bruteforce.layer(geom, w.conv_w, w.A_log, w.dt_bias, w.norm_w,
                                      x, z, a, b, S0, W0)
    np.testing.assert_allclose(o, ob, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(y, yb, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(S, Sb, rtol=1e-11, atol=1e-12)
    np.testing.assert_array_equal(W, Wb)


@pytest.mark.parametrize("chunk,T,slow", [(64, 150, False), (16, 70, True), (7, 30, False),
                                          (64, 64, True), (64, 1, False)])
def test_chunkwise_equals_token_loop(chunk, T, slow):
    rng = np.random.default_rng(20 + chunk + T)
    geom = oracle.Geometry(2, 4, 16, 12, 4)
    w, x, z, a, b, S0, W0 = _rand_layer(rng, geom, T)
    if slow:
        w.A_log[:] = np.log(rng.uniform(0.002, 0.03, geom.num_v_heads))
    else:
        w.A_log[:] = np.log(rng.uniform(1, 16, geom.num_v_heads))   # g down to ~ -80
        a[:5] += 4.0
    y0, o0, S_0, _ = _run(geom, w, x, z, a, b, S0, W0)
    y1, o1, S_1, _ = _run(geom, w, x, z, a, b, S0, W0, chunk=chunk)
    scale = np.abs(o0).max()
    assert np.abs(o1 - o0).max() <= 1e-12 * scale
    assert np.abs(S_1 - S_0).max() <= 1e-12 * np.abs(S_0).max()
    assert np.abs(y1 - y0).max() <= 1e-10 * np.abs(y0).max()


def test_value_columns_evolve_independently():
    """Splitting dv in halves gives the same state columns and outputs."""
    rng = np.random.default_rng(30)
    Hk, Hv, dk, dv, K = 2, 4, 6, 8, 4
    full = oracle.Geometry(Hk, Hv, dk, dv, K)
    half = oracle.Geometry(Hk, Hv, dk, dv // 2, K)
    w, x, z, a, b, S0, W0 = _rand_layer(rng, full, 12)
    _, o, S, _ = _run(full, w, x, z, a, b, S0, W0)
    for part in range(2):
        cols = slice(part * dv // 2, (part + 1) * dv // 2)
        vch = np.concatenate([2 * Hk * dk + h * dv + np.arange(dv)[cols] for h in range(Hv)])
        ch = np.concatenate([np.arange(2 * Hk * dk), vch])
        wh = oracle.Weights(w.conv_w[ch], w.A_log, w.dt_bias, w.norm_w[cols])
        _, oh, Sh, _ = _run(half, wh, x[:, ch], z[:, :, cols], a, b, S0[:, :, cols],
                            W0[:, ch])
        np.testing.assert_allclose(oh, o[:, :, cols], rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(Sh, S[:, :, cols], rtol=1e-13, atol=1e-15)


def test_gqa_is_repeat_interleave():
    """V-heads 0 and 1 read K-head 0 (repeat_interleave), not heads 0 and 2."""
    rng = np.random.default_rng(31)
    geom = oracle.Geometry(2, 4, 6, 5, 4)
    w, x, z, a, b, S0, W0 = _rand_layer(rng, geom, 9)
    v0 = 2 * 2 * 6
    for h in (1, 2):   # copy head 0's value channels, weights, gates and state
        x[:, v0 + h * 5: v0 + (h + 1) * 5] = x[:, v0: v0 + 5]
        W0[:, v0 + h * 5: v0 + (h + 1) * 5] = W0[:, v0: v0 + 5]
        w.conv_w[v0 + h * 5: v0 + (h + 1) * 5] = w.conv_w[v0: v0 + 5]
        w.A_log[h], w.dt_bias[h] = w.A_log[0], w.dt_bias[0]
        a[:, h], b[:, h], S0[h] = a[:, 0], b[:, 0], S0[0]
    _, o, S, _ = _run(geom, w, x, z, a, b, S0, W0)
    np.testing.assert_array_equal(o[:, 1], o[:, 0])
    np.testing.assert_array_equal(S[1], S[0])
    assert np.abs(o[:, 2] - o[:, 0]).max() > 1e-3


# ------------------------------------------------------------ gated norm


def test_gated_rmsnorm_matches_torch():
    rng = np.random.default_rng(40)
    o, z, w = rng.normal(size=16), rng.normal(size=16), 1 + 0.1 * rng.normal(size=16)
    got = oracle.gated_rmsnorm(o, z, w, 1e-6)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(o), (16,), torch.from_numpy(w), 1e-6)
    ref = (ref * torch.nn.functional.silu(torch.from_numpy(z))).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-14, atol=1e-15)
    # normalised: mean((y / (w silu z))^2) -> 1 for |o| >> sqrt(eps)
    r = got / (w * z / (1 + np.exp(-z)))
    assert abs(np.mean(r * r) - 1) < 1e-5


# ------------------------------------------------------------ slot pool


def _pool_case(seed, P=6, B=4):
    rng = np.random.default_rng(seed)
    w, x, z, a, b, _, _ = _rand_layer(rng, G, B)
    pS = rng.normal(0, 0.1, (P, G.num_v_heads, G.head_k_dim, G.head_v_dim))
    pC = rng.normal(0, 0.1, (P, G.conv_kernel, G.channels))
    return rng, w, x, z, a, b, pS, pC


def test_decode_rows_padding_and_untouched_slots():
    rng, w, x, z, a, b, pS, pC = _pool_case(50)
    slots = np.array([4, -1, 0, 2], np.int32)
    S1, C1 = pS.copy(), pC.copy()
    y, o = oracle.pool_run(G, w, S1, C1, np.arange(5), slots, x, z, a, b)
    assert not y[1].any() and not o[1].any()
    for s in (1, 3, 5):
        np.testing.assert_array_equal(S1[s], pS[s])
        np.testing.assert_array_equal(C1[s], pC[s])
    for row, s in ((0, 4), (2, 0), (3, 2)):
        yy, oo, SS, WW = _run(G, w, x[row:row + 1], z[row:row + 1], a[row:row + 1],
                              b[row:row + 1], pS[s], pC[s])
        np.testing.assert_array_equal(y[row], yy[0])
        np.testing.assert_array_equal(S1[s], SS)
        np.testing.assert_array_equal(C1[s], WW)


def test_row_permutation_permutes_outputs():
    rng, w, x, z, a, b, pS, pC = _pool_case(51)
    slots = np.array([3, 1, 5, 0], np.int32)
    perm = np.array([2, 0, 3, 1])
    S1, C1, S2, C2 = pS.copy(), pC.copy(), pS.copy(), pC.copy()
    y1, _ = oracle.pool_run(G, w, S1, C1, np.arange(5), slots, x, z, a, b)
    y2, _ = oracle.pool_run(G, w, S2, C2, np.arange(5), slots[perm], x[perm], z[perm],
                            a[perm], b[perm])
    np.testing.assert_array_equal(y2, y1[perm])
    np.testing.assert_array_equal(S2, S1)
    np.testing.assert_array_equal(C2, C1)


def test_prefill_then_decode_equals_longer_prefill():
    rng = np.random.default_rng(52)
    w, x, z, a, b, _, _ = _rand_layer(rng, G, 20)
    pS = np.zeros((1, G.num_v_heads, G.head_k_dim, G.head_v_dim))
    pC = np.zeros((1, G.conv_kernel, G.channels))
    S1, C1 = pS.copy(), pC.copy()
    y_all, _ = oracle.pool_run(G, w, S1, C1, [0, 20], [0], x, z, a, b)
    S2, C2 = pS.copy(), pC.copy()
    y_pre, _ = oracle.pool_run(G, w, S2, C2, [0, 14], [0], x[:14], z[:14], a[:14], b[:14])
    ys = [y_pre]
    for t in range(14, 20):
        yt, _ = oracle.pool_run(G, w, S2, C2, [0, 1], [0], x[t:t + 1], z[t:t + 1],
                                a[t:t + 1], b[t:t + 1])
        ys.append(yt)
    np.testing.assert_allclose(np.concatenate(ys), y_all, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(S2, S1, rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(C2, C1)


def test_packed_sequences_equal_separate_runs_and_has_init():
    rng = np.random.default_rng(53)
    lens = [5, 1, 9]
    cu = np.concatenate([[0], np.cumsum(lens)])
    w, x, z, a, b, _, _ = _rand_layer(rng, G, int(cu[-1]))
    pS = rng.normal(0, 0.1, (4, G.num_v_heads, G.head_k_dim, G.head_v_dim))
    pC = rng.normal(0, 0.1, (4, G.conv_kernel, G.channels))
    slots = np.array([2, 0, 3], np.int32)
    init = np.array([1, 0, 1], np.uint8)
    S1, C1 = pS.copy(), pC.copy()
    y, _ = oracle.pool_run(G, w, S1, C1, cu, slots, x, z, a, b, has_init=init)
    for n in range(3):
        sl = slice(cu[n], cu[n + 1])
        s0 = pS[slots[n]] if init[n] else np.zeros_like(pS[0])
        w0 = pC[slots[n]] if init[n] else np.zeros_like(pC[0])
        yy, _, SS, WW = _run(G, w, x[sl], z[sl], a[sl], b[sl], s0, w0)
        np.testing.assert_array_equal(y[sl], yy)
        np.testing.assert_array_equal(S1[slots[n]], SS)
        np.testing.assert_array_equal(C1[slots[n]], WW)
    np.testing.assert_array_equal(S1[1], pS[1])


def test_compaction_copies_slots():
    rng = np.random.default_rng(54)
    pS = rng.normal(size=(6, G.num_v_heads, G.head_k_dim, G.head_v_dim))
    pC = rng.normal(size=(6, G.conv_kernel, G.channels))
    S1, C1 = pS.copy(), pC.copy()
    oracle.compact(G, S1, C1, [4, 5], [0, 2])
    np.testing.assert_array_equal(S1[[0, 2]], pS[[4, 5]])
    np.testing.assert_array_equal(C1[[0, 2]], pC[[4, 5]])
    np.testing.assert_array_equal(S1[[1, 3, 4, 5]], pS[[1, 3, 4, 5]])


def test_workload_generator_uses_bf16_grid():
    s = Shape(2, 4, 8, 8, 4, "bf16")
    rng = np.random.default_rng(0)
    w = layer_weights(rng, s)
    inp = token_inputs(rng, s, 3)
    for arr in (w["conv_w"], inp["x"], inp["z"]):
        t = torch.from_numpy(arr)
        assert torch.equal(t.to(torch.bfloat16).to(torch.float32), t)


# ------------------------------------------------------------------ projections

def test_linear_matches_loops_on_non_square():
    """y[m][n] = sum_k x[m][k] w[n][k] with w stored [out][in]: brute-force
    loops on a 3 x 5 input and a 4 x 5 weight (a transposed operand or a
    swapped product changes the shape or the values)."""
    rng = np.random.default_rng(7)
    x = rng.integers(-4, 5, (3, 5)).astype(np.float64)
    w = rng.integers(-4, 5, (4, 5)).astype(np.float64)
    ref = [[sum(x[m][k] * w[n][k] for k in range(5)) for n in range(4)] for m in range(3)]
    y = oracle.linear(x, w)
    assert y.shape == (3, 4)
    np.testing.assert_array_equal(y, np.array(ref))


def test_block_with_selection_projections_is_the_layer():
    """With input projections that pick disjoint ranges of the hidden row and
    an out_proj that copies y into the first Hv*dv outputs, the block equals
    the layer run on those ranges as x, z, b, a (in that order), and the
    remaining outputs are zero.  Pins which projection feeds which input."""
    rng = np.random.default_rng(11)
    C, Hv, dv = G.channels, G.num_v_heads, G.head_v_dim
    vd = Hv * dv
    H = C + vd + 2 * Hv
    E = np.eye(H)
    out = np.zeros((H, vd))
    out[:vd] = np.eye(vd)
    proj = oracle.Projections(qkv=E[:C], z=E[C:C + vd], b=E[C + vd:C + vd + Hv],
                              a=E[C + vd + Hv:], out=out)
    w, *_ = _rand_layer(rng, G, 1)
    B, P = 5, 8
    S = rng.normal(0, 0.3, (P, Hv, G.head_k_dim, dv))
    W = rng.normal(size=(P, G.conv_kernel, C))
    slots = rng.choice(P, B, replace=False).astype(np.int32)
    h = rng.normal(size=(B, H))
    S1, W1 = S.copy(), W.copy()
    got, inp, y = oracle.decode_block(G, w, proj, S1, W1, slots, h)
    S2, W2 = S.copy(), W.copy()
    y_ref, _ = oracle.pool_run(G, w, S2, W2, np.arange(B + 1), slots, h[:, :C],
                               h[:, C:C + vd].reshape(B, Hv, dv), h[:, C + vd + Hv:],
                               h[:, C + vd:C + vd + Hv])
    np.testing.assert_array_equal(y, y_ref)
    np.testing.assert_array_equal(got[:, :vd], y_ref.reshape(B, vd))
    assert not got[:, vd:].any()
    np.testing.assert_array_equal(S1, S2)
    np.testing.assert_array_equal(W1, W2)
    np.testing.assert_array_equal(inp["a"], h[:, C + vd + Hv:])
