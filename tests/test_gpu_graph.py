"""Calls captured in a HIP graph and replayed give the same bits as the same
calls launched one by one (the decode path the bench times runs from graph
replays).  Each replay is checked, with eager work between replays, and the
device slot index is rewritten in place between replays as the serving loop
does.  The fused decode step's workgroups meet through counters in the
caller's workspace, but every value they compute is the same whichever
arrives last (each sum is formed in a fixed order), so the comparison is
exact."""
import numpy as np
import pytest
import torch

import linear_attention_causal_amd as gdn
import workloads as wl
from gpu_helpers import DEV, Layer, Pool, ServingRows, dev, host

pytestmark = pytest.mark.gpu


def _capture(fn):
    """Capture fn() on a side stream into a graph.  fn allocates nothing (its
    buffers exist beforehand) and capturing runs none of its kernels."""
    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            fn()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    return graph


def test_decode_steps_graph_replay_matches_eager():
    work = wl.decode_batch(seed=21, B=16, P=64)
    s, d = work.shape, work.data
    print(f"[graph] {work.name}", flush=True)
    L = Layer(s, d["weights"])
    rng = np.random.default_rng(5)
    steps = [wl.token_inputs(rng, s, 16) for _ in range(3)]
    act = torch.bfloat16
    ins = [{k: dev(t[k], act) for k in ("x", "z", "a", "b")} for t in steps]
    y_g = [torch.empty(16, s.num_v_heads, s.head_v_dim, device=DEV, dtype=act) for _ in steps]
    y_e = [torch.empty_like(y) for y in y_g]
    Pg, Pe = Pool(s, d["rec"], d["conv"]), Pool(s, d["rec"], d["conv"])
    slot_g = dev(d["slot_idx"], torch.int32)
    slot_e = dev(d["slot_idx"], torch.int32)
    ws_g, ws_e = gdn.decode_workspace(L.geom, 16), gdn.decode_workspace(L.geom, 16)

    def run(pool, slot, ys, ws):
        for t, y in zip(ins, ys):
            gdn.gdn_decode_step(L.geom, L.w, pool.pool, slot, t["x"], t["z"], t["a"], t["b"], y,
                                ws)

    graph = _capture(lambda: run(Pg, slot_g, y_g, ws_g))
    perm = np.random.default_rng(9)
    for rep in range(3):
        if rep > 0:   # rows move to other slots between replays (in place)
            new = perm.choice(64, 16, replace=False).astype(np.int32)
            new[rep] = -1   # and one row is padding
            slot_g.copy_(dev(new, torch.int32))
            slot_e.copy_(dev(new, torch.int32))
        graph.replay()
        run(Pe, slot_e, y_e, ws_e)
        torch.cuda.synchronize()
        for i in range(len(ins)):
            assert torch.equal(y_g[i], y_e[i]), f"replay {rep}: y of step {i} differs"
        assert torch.equal(Pg.rec, Pe.rec), f"replay {rep}: recurrent pool differs"
        assert torch.equal(Pg.conv, Pe.conv), f"replay {rep}: conv pool differs"


def test_decode_block_graph_replay_matches_eager():
    work = wl.decode_block(seed=4, B=16, P=64)
    s, d = work.shape, work.data
    print(f"[graph] {work.name}", flush=True)
    L = Layer(s, d["weights"])
    bf = torch.bfloat16
    proj = {k: dev(v, bf) for k, v in d["proj"].items()}
    B, H = d["hidden"].shape
    C, vd, Hv = s.channels, s.num_v_heads * s.head_v_dim, s.num_v_heads

    def buffers():
        return dict(qkv=torch.empty(B, C, device=DEV, dtype=bf),
                    z=torch.empty(B, vd, device=DEV, dtype=bf),
                    b=torch.empty(B, Hv, device=DEV, dtype=bf),
                    a=torch.empty(B, Hv, device=DEV, dtype=bf),
                    y=torch.empty(B, vd, device=DEV, dtype=bf),
                    out=torch.empty(B, H, device=DEV, dtype=bf))

    h = dev(d["hidden"], bf)
    slot = dev(d["slot_idx"], torch.int32)
    ws = gdn.decode_workspace(L.geom, B)
    bg, be = buffers(), buffers()
    Pg, Pe = Pool(s, d["rec"], d["conv"]), Pool(s, d["rec"], d["conv"])

    def block(pool, o):
        gdn.gdn_linear(h, [(proj["qkv"], o["qkv"]), (proj["z"], o["z"]), (proj["b"], o["b"]),
                           (proj["a"], o["a"])])
        gdn.gdn_decode_step(L.geom, L.w, pool.pool, slot, o["qkv"], o["z"], o["a"], o["b"],
                            o["y"], ws)
        gdn.gdn_linear(o["y"], [(proj["out"], o["out"])])

    graph = _capture(lambda: block(Pg, bg))
    for rep in range(3):
        graph.replay()
        block(Pe, be)
        torch.cuda.synchronize()
        for k in bg:
            assert torch.equal(bg[k], be[k]), f"replay {rep}: {k} differs"
        assert torch.equal(Pg.rec, Pe.rec) and torch.equal(Pg.conv, Pe.conv), f"replay {rep}"


def test_prefill_graph_replay_matches_eager():
    s = wl.Shape(2, 4, 64, 64, 4, "bf16")
    rng = np.random.default_rng(12)
    w = wl.layer_weights(rng, s)
    lens = [130, 64, 1, 200]
    T = sum(lens)
    inp = wl.token_inputs(rng, s, T)
    rec, conv = wl.state_pool(rng, s, 6)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    slots = np.array([4, 0, 2, 5], np.int32)
    print(f"[graph] prefill lengths {lens}", flush=True)
    L = Layer(s, w)
    act = torch.bfloat16
    x, z, a, b = (dev(inp[k], act) for k in ("x", "z", "a", "b"))
    cu_d = dev(cu, torch.int32)
    sl = dev(slots, torch.int32)
    nbytes = gdn.gdn_prefill_scratch_bytes(L.geom, T, len(lens))
    y_g = torch.empty(T, s.num_v_heads, s.head_v_dim, device=DEV, dtype=act)
    y_e = torch.empty_like(y_g)
    scr_g = torch.empty(nbytes, device=DEV, dtype=torch.uint8)
    scr_e = torch.empty(nbytes, device=DEV, dtype=torch.uint8)
    Pg, Pe = Pool(s, rec, conv), Pool(s, rec, conv)
    rec0, conv0 = Pe.rec.clone(), Pe.conv.clone()

    def call(pool, y, scr):
        gdn.gdn_prefill_chunked(L.geom, L.w, pool.pool, cu, cu_d, sl, x, z, a, b, y, scr,
                                slot_idx_host=slots)

    graph = _capture(lambda: call(Pg, y_g, scr_g))
    for rep in range(2):
        # every replay starts from the initial pools, as does the eager call
        Pg.rec.copy_(rec0)
        Pg.conv.copy_(conv0)
        Pe.rec.copy_(rec0)
        Pe.conv.copy_(conv0)
        graph.replay()
        call(Pe, y_e, scr_e)
        torch.cuda.synchronize()
        assert torch.equal(y_g, y_e), f"replay {rep}: y differs"
        assert torch.equal(Pg.rec, Pe.rec) and torch.equal(Pg.conv, Pe.conv), f"replay {rep}"


def test_bucketed_graph_replay_matches_oracle():
    """Serving by replay only, one captured graph per batch bucket: the
    decode steps of three layers are captured once for a 32-row and once for
    a 64-row bucket (pegainfer issue #1001, Splits, "TP CUDA Graph": a
    pre-capture sweep per bucket and replay-only serving).  The live rows are
    padded up to the smallest bucket that holds them (padding rows carry slot
    -1 and get zero outputs); before each replay the bucket's slot index and
    input buffers are rewritten in place.  Retire events compact the pools of
    all layers and change the bucket both ways (50 rows -> 27 -> 44).  The
    replayed y of every live row and every layer's final states are compared
    with the oracle."""
    s = wl.RANK_LOCAL
    layers, P, buckets = 3, 80, (32, 64)
    rng = np.random.default_rng(17)
    wts = [wl.layer_weights(rng, s) for _ in range(layers)]
    init = [wl.state_pool(rng, s, P) for _ in range(layers)]
    print(f"[graph] buckets {buckets}, {layers} layers", flush=True)
    Ls = [Layer(s, w) for w in wts]
    Ps = [Pool(s, *init[l]) for l in range(layers)]
    rows = ServingRows(rng.choice(P, 50, replace=False).astype(np.int32))
    bf = torch.bfloat16
    C, Hv, dv = s.channels, s.num_v_heads, s.head_v_dim
    bk = {}
    for Bk in buckets:
        b = dict(x=torch.zeros(Bk, C, device=DEV, dtype=bf),
                 z=torch.zeros(Bk, Hv, dv, device=DEV, dtype=bf),
                 a=torch.zeros(Bk, Hv, device=DEV, dtype=bf),
                 b=torch.zeros(Bk, Hv, device=DEV, dtype=bf),
                 y=torch.empty(Bk, Hv, dv, device=DEV, dtype=bf),
                 slot=torch.full((Bk,), -1, device=DEV, dtype=torch.int32),
                 ws=gdn.decode_workspace(Ls[0].geom, Bk))

        def step(b=b):
            for L, Pl in zip(Ls, Ps):
                gdn.gdn_decode_step(L.geom, L.w, Pl.pool, b["slot"], b["x"], b["z"], b["a"],
                                    b["b"], b["y"], b["ws"])
        b["graph"] = _capture(step)
        bk[Bk] = b
    used = []
    for t in range(10):
        if t in (4, 7):
            src, dst, free = rows.retire(rng, P, n_admit=2 if t == 4 else 30)
            gdn.gdn_state_compact(Ls[0].geom, [p.pool for p in Ps], src, dst,
                                  dev(src, torch.int32), dev(dst, torch.int32))
            for p in Ps:
                p.rec[free] = 0
                p.conv[free] = 0
        n = len(rows.active)
        Bk = min(x for x in buckets if x >= n)
        used.append(Bk)
        b = bk[Bk]
        inp = wl.token_inputs(rng, s, n)
        for k in ("x", "z", "a", "b"):
            b[k][:n].copy_(dev(inp[k], bf))
        b["slot"].fill_(-1)
        b["slot"][:n].copy_(dev(rows.live_slots(), torch.int32))
        b["graph"].replay()
        yh = host(b["y"])
        assert not yh[n:].any(), f"step {t}: padding rows not zero"
        rows.record(inp, yh[:n])
    assert set(used) == set(buckets), used
    rows.check(Ls, Ps, init, s, tag="bucketed graph replay")
    for b in bk.values():
        assert not b["ws"].any()
