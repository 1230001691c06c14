"""GPU state compaction (gdn_state_compact): a bit-exact copy of whole slots
across every layer, nothing else touched; and decode schedules with retire /
compact / admit whose live rows all match the oracle's per-sequence results,
up to the full-head serving shape."""
import numpy as np
import pytest
import torch

import linear_attention_causal_amd as gdn
import workloads as wl
from gpu_helpers import Layer, Pool, ServingRows, decode_step, dev, host

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
    """B=48 rows of a 64-slot pool, 2 layers, 24 steps of the two-call decode
    (gdn_conv_update + gdn_decode_batch); after steps 8 and 16 a seeded half
    of the rows retire, survivors are compacted by hole filling and new rows
    are admitted with zero state.  Every live row at the end is compared with
    the oracle running its tokens as one sequence."""
    s = wl.Shape(4, 8, 64, 64, 4, "bf16")
    rng = np.random.default_rng(11)
    P, B0, steps, layers = 64, 48, 24, 2
    ws = [wl.layer_weights(rng, s) for _ in range(layers)]
    init = [wl.state_pool(rng, s, P) for _ in range(layers)]
    Ls = [Layer(s, w) for w in ws]
    Ps = [Pool(s, *init[l]) for l in range(layers)]
    rows = ServingRows(rng.choice(P, B0, replace=False).astype(np.int32))
    for t in range(steps):
        if t in (8, 16):
            src, dst, free = rows.retire(rng, P)
            if src.size:
                gdn.gdn_state_compact(Ls[0].geom, [p.pool for p in Ps], src, dst,
                                      dev(src, torch.int32), dev(dst, torch.int32))
            for p in Ps:   # admitted rows start from zero state
                p.rec[free] = 0
                p.conv[free] = 0
        inp = wl.token_inputs(rng, s, len(rows.active))
        sl = rows.live_slots()
        for l in range(layers):
            y, _ = decode_step(Ls[l], Ps[l], sl, inp["x"], inp["z"], inp["a"], inp["b"],
                               want_o=False)
        rows.record(inp, host(y))
    rows.check(Ls, Ps, init, s, tag="two-call schedule")


def test_serving_schedule_full_heads():
    """The full-head serving shape: Hk=16, Hv=32, d=128, B=256 rows of a
    320-slot pool, two layers run by the fused step with a device-resident
    slot index and no host copy (as a replayed graph runs it), nine steps
    with a retire event after steps 3 and 6: a seeded half of the rows
    retire, survivors are compacted into the prefix by hole filling
    (gdn_state_compact over both layers), new rows are admitted behind them
    with zeroed state, and the device slot index is rewritten in place.
    Every live row at the end (all 256) is checked against the oracle: both
    layers' states and conv windows and the last layer's y for every token."""
    s = wl.FULL_HEADS
    rng = np.random.default_rng(13)
    P, B, steps, layers = 320, 256, 9, 2
    ws = [wl.layer_weights(rng, s) for _ in range(layers)]
    init = [wl.state_pool(rng, s, P) for _ in range(layers)]
    print(f"[schedule] full heads B={B} P={P} layers={layers} steps={steps}", flush=True)
    Ls = [Layer(s, w) for w in ws]
    Ps = [Pool(s, *init[l]) for l in range(layers)]
    rows = ServingRows(rng.choice(P, B, replace=False).astype(np.int32))
    slot_d = dev(rows.live_slots(), torch.int32)
    wsp = gdn.decode_workspace(Ls[0].geom, B)
    bf = torch.bfloat16
    y = torch.empty(B, s.num_v_heads, s.head_v_dim, device="cuda", dtype=bf)
    for t in range(steps):
        if t in (3, 6):
            src, dst, free = rows.retire(rng, P)
            gdn.gdn_state_compact(Ls[0].geom, [p.pool for p in Ps], src, dst,
                                  dev(src, torch.int32), dev(dst, torch.int32))
            for p in Ps:
                p.rec[free] = 0
                p.conv[free] = 0
            slot_d.copy_(dev(rows.live_slots(), torch.int32))
            print(f"  step {t}: {src.size} slots moved, {len(free)} admitted", flush=True)
        inp = wl.token_inputs(rng, s, B)
        x, z, a, b = (dev(inp[k], bf) for k in ("x", "z", "a", "b"))
        for l in range(layers):
            gdn.gdn_decode_step(Ls[l].geom, Ls[l].w, Ps[l].pool, slot_d, x, z, a, b, y, wsp)
        rows.record(inp, host(y))
    rows.check(Ls, Ps, init, s, tag="full-head schedule")
    assert not wsp.any()
