"""GPU state compaction (gdn_state_compact): a bit-exact copy of whole slots
across every layer, nothing else touched; and a decode schedule with retire /
compact / admit whose sampled rows still match the oracle's per-sequence
results."""
import numpy as np
import pytest
import torch

import linear_attention_causal_amd as gdn
import oracle
import workloads as wl
from gpu_helpers import (TOL_F32, Layer, Pool, assert_close, decode_step, dev, host,
                         maxrel_heads, maxrel_states, y_tol)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("shape,L", [(wl.RANK_LOCAL, 3), (wl.TINY, 40)])
def test_compaction_is_bitwise_copy(shape, L):
    rng = np.random.default_rng(0)
    P = 12
    pools = [Pool(shape, *wl.state_pool(rng, shape, P)) for _ in range(L)]
    before = [(host(p.rec), host(p.conv)) for p in pools]
    src = np.array([9, 11, 7], np.int32)
    dst = np.array([1, 4, 2], np.int32)
    geom = Layer(shape, wl.layer_weights(rng, shape)).geom
    gdn.gdn_state_compact(geom, [p.pool for p in pools], src, dst, dev(src, torch.int32),
                          dev(dst, torch.int32))
    for p, (r0, c0) in zip(pools, before):
        r1, c1 = host(p.rec), host(p.conv)
        exp_r, exp_c = r0.copy(), c0.copy()
        exp_r[dst], exp_c[dst] = r0[src], c0[src]
        np.testing.assert_array_equal(r1, exp_r)
        np.testing.assert_array_equal(c1, exp_c)


def test_decode_schedule_with_retire_and_compaction():
    """B=48 rows of a 64-slot pool, 2 layers, 24 steps; after steps 8 and 16 a
    seeded half of the rows retire, survivors are compacted by hole filling
    and new rows are admitted with zero state.  Sampled surviving rows are
    compared with the oracle running each row's tokens as one sequence."""
    s = wl.Shape(4, 8, 64, 64, 4, "bf16")
    rng = np.random.default_rng(11)
    P, B0, steps, layers = 64, 48, 24, 2
    ws = [wl.layer_weights(rng, s) for _ in range(layers)]
    init = [wl.state_pool(rng, s, P) for _ in range(layers)]
    Ls = [Layer(s, w) for w in ws]
    Ps = [Pool(s, *init[l]) for l in range(layers)]
    slots0 = rng.choice(P, B0, replace=False).astype(np.int32)
    # logical rows: initial slot (None = admitted fresh), tokens seen, last-layer y
    rows = [dict(start=int(sl), toks=[]) for sl in slots0]
    active = list(range(B0))
    slot_of = {i: int(slots0[i]) for i in active}
    for t in range(steps):
        if t in (8, 16):
            live = np.array([slot_of[i] for i in active], np.int32)
            keep, new_slots, src, dst = wl.retire_plan(rng, live, P)
            if src.size:
                gdn.gdn_state_compact(Ls[0].geom, [p.pool for p in Ps], src, dst,
                                      dev(src, torch.int32), dev(dst, torch.int32))
            survivors = [i for i, k in zip(active, keep) if k]
            for i, ns in zip(survivors, new_slots):
                slot_of[i] = int(ns)
            n_new = len(active) - len(survivors)
            free = list(range(len(survivors), len(survivors) + n_new))
            for p in Ps:   # admitted rows start from zero state
                p.rec[free] = 0
                p.conv[free] = 0
            for f in free:
                rows.append(dict(start=None, toks=[]))
                slot_of[len(rows) - 1] = f
            active = survivors + list(range(len(rows) - n_new, len(rows)))
        inp = wl.token_inputs(rng, s, len(active))
        sl = np.array([slot_of[i] for i in active], np.int32)
        for l in range(layers):
            y, _ = decode_step(Ls[l], Ps[l], sl, inp["x"], inp["z"], inp["a"], inp["b"],
                               want_o=False)
        yh = host(y)
        for j, i in enumerate(active):
            rows[i]["toks"].append({k: inp[k][j] for k in inp} | {"y": yh[j]})
    sample = active[:: max(1, len(active) // 6)]
    for i in sample:
        r = rows[i]
        tok = {k: np.stack([t[k] for t in r["toks"]]) for k in ("x", "z", "a", "b")}
        T = len(r["toks"])
        for l in range(layers):
            if r["start"] is None:
                S0 = np.zeros((1, s.num_v_heads, s.head_k_dim, s.head_v_dim))
                W0 = np.zeros((1, s.conv_kernel, s.channels))
            else:
                S0 = init[l][0][r["start"]][None].astype(np.float64)
                W0 = init[l][1][r["start"]][None].astype(np.float64)
            yo, _, Sn, Wn = oracle.sequences(Ls[l].og, Ls[l].ow, [0, T], tok["x"], tok["z"],
                                             tok["a"], tok["b"], S0, W0)
            assert_close(f"row {i} layer {l} state",
                         maxrel_states(host(Ps[l].rec)[slot_of[i]], Sn[0]), TOL_F32)
            np.testing.assert_array_equal(host(Ps[l].conv)[slot_of[i]], Wn[0])
            if l == layers - 1:
                ygpu = np.stack([t["y"] for t in r["toks"]])
                assert_close(f"row {i} y", maxrel_heads(ygpu, yo), y_tol(s))
