"""Independent numpy form of the Gated DeltaNet layer for tiny shapes.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Written separately from gdn_oracle.c so that the two can check each other:
  * the conv is a sliding-window product over the concatenated stream;
  * the recurrence uses its transition-matrix form,
        S_t = e^{g_t} (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,
    with explicit dk x dk matrices, which is the gated delta rule
    S_t = e^{g_t} S_{t-1} + beta_t k_t (v_t - e^{g_t} S_{t-1}^T k_t)^T
    multiplied out (Yang, Kautz & Hatamizadeh, "Gated Delta Networks",
    ICLR 2025; the per-V-head delta-rule state of cortex commit 95dc874,
    TpQwen3_5GatedDeltaNet bullet);
  * the gates and norms are written from their closed forms.
"""
import numpy as np


def layer(geom, conv_w, A_log, dt_bias, norm_w, x, z, a, b, S0, window0):
    """One sequence.  x [T][C], z [T][Hv][dv], a/b [T][Hv], S0 [Hv][dk][dv],
    window0 [K][C].  Returns y, o [T][Hv][dv], S [Hv][dk][dv], window [K][C]."""
    Hk, Hv = geom.num_k_heads, geom.num_v_heads
    dk, dv, K = geom.head_k_dim, geom.head_v_dim, geom.conv_kernel
    x = np.asarray(x, np.float64)
    T, C = x.shape
    stream = np.concatenate([np.asarray(window0, np.float64), x], axis=0)  # [K+T][C]
    # token t sees stream rows t+1 .. t+K; tap j multiplies row t+1+j
    win = np.lib.stride_tricks.sliding_window_view(stream[1:], K, axis=0)  # [T][C][K]
    pre = np.einsum("tck,ck->tc", win[:T], np.asarray(conv_w, np.float64))
    act = pre / (1.0 + np.exp(-pre))
    q = act[:, : Hk * dk].reshape(T, Hk, dk)
    k = act[:, Hk * dk: 2 * Hk * dk].reshape(T, Hk, dk)
    v = act[:, 2 * Hk * dk:].reshape(T, Hv, dv)
    scale = geom.scale if geom.scale > 0 else dk ** -0.5
    qn = q / np.sqrt((q * q).sum(-1, keepdims=True) + geom.l2norm_eps) * scale
    kn = k / np.sqrt((k * k).sum(-1, keepdims=True) + geom.l2norm_eps)
    sp = np.logaddexp(0.0, np.asarray(a, np.float64) + np.asarray(dt_bias, np.float64))
    g = -np.exp(np.asarray(A_log, np.float64)) * sp            # [T][Hv]
    beta = 1.0 / (1.0 + np.exp(-np.asarray(b, np.float64)))    # [T][Hv]
    r = Hv // Hk
    S = np.array(S0, np.float64, copy=True)
    o = np.zeros((T, Hv, dv))
    eye = np.eye(dk)
    for t in range(T):
        for h in range(Hv):
            kk = kn[t, h // r]
            M = np.exp(g[t, h]) * (eye - beta[t, h] * np.outer(kk, kk))
            S[h] = M @ S[h] + beta[t, h] * np.outer(kk, v[t, h])
            o[t, h] = S[h].T @ qn[t, h // r]
    rms = np.sqrt((o * o).mean(-1, keepdims=True) + geom.rmsnorm_eps)
    zz = np.asarray(z, np.float64)
    y = np.asarray(norm_w, np.float64) * o / rms * (zz / (1.0 + np.exp(-zz)))
    window = stream[-K:].copy()
    return y, o, S, window
