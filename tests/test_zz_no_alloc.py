"""gdn_decode_step_noalloc (the decode step on the library-held workspace)
against gdn_decode_step with a caller workspace and against the oracle:
two calls in a row on the same pools, the second with fewer rows, each
checked; the same kernel runs either way, so outputs and pools are compared
bit for bit, and y / o_raw / states against the f64 oracle."""
import numpy as np
import pytest
import torch

import linear_attention_causal_amd as gdn
import oracle
import workloads as wl
from gpu_helpers import (TOL_F32, Layer, Pool, act_dtype, assert_close, dev, host, maxrel_heads,
                         maxrel_states, y_tol)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("s,sizes", [(wl.RANK_LOCAL, (16, 5)), (wl.FULL_HEADS, (256, 40)),
                                     (wl.TINY, (9, 2))])
def test_noalloc_step_matches_workspace_step(s, sizes):
    P = max(sizes) + 8
    work = wl.decode_batch(seed=77, B=4, P=P, s=s)
    d = work.data
    print(f"[noalloc] {work.name} rows {sizes}", flush=True)
    L = Layer(s, d["weights"])
    Pn, Pw = Pool(s, d["rec"], d["conv"]), Pool(s, d["rec"], d["conv"])
    S, W = d["rec"].astype(np.float64), d["conv"].astype(np.float64)
    ws = gdn.decode_workspace(L.geom, max(sizes))
    rng = np.random.default_rng(78)
    ad = act_dtype(s)
    for call, B in enumerate(sizes):
        slots = rng.choice(P, B, replace=False).astype(np.int32)
        slots[B // 2] = -1
        inp = wl.token_inputs(rng, s, B)
        x, z, a, b = (dev(inp[k], ad) for k in ("x", "z", "a", "b"))
        sl = dev(slots, torch.int32)
        shape = (B, s.num_v_heads, s.head_v_dim)
        yn, yw = torch.empty(shape, device="cuda", dtype=ad), torch.empty(shape, device="cuda", dtype=ad)
        on, ow = torch.empty(shape, device="cuda"), torch.empty(shape, device="cuda")
        gdn.gdn_decode_step_noalloc(L.geom, L.w, Pn.pool, sl, x, z, a, b, yn, o_raw=on)
        gdn.gdn_decode_step(L.geom, L.w, Pw.pool, sl, x, z, a, b, yw, ws, o_raw=ow)
        torch.cuda.synchronize()
        assert torch.equal(yn, yw) and torch.equal(on, ow), f"call {call}: outputs differ"
        assert torch.equal(Pn.rec, Pw.rec) and torch.equal(Pn.conv, Pw.conv), f"call {call}: pools"
        keep = slots >= 0
        yo, oo = oracle.pool_run(L.og, L.ow, S, W, np.arange(keep.sum() + 1), slots[keep],
                                 *(inp[k][keep] for k in ("x", "z", "a", "b")))
        assert_close(f"call {call} (B={B}) y", maxrel_heads(host(yn)[keep], yo), y_tol(s))
        assert_close(f"call {call} (B={B}) o_raw", maxrel_heads(host(on)[keep], oo), TOL_F32)
        assert not host(yn)[~keep].any()
    assert_close("states", maxrel_states(host(Pn.rec), S), TOL_F32)
    np.testing.assert_array_equal(host(Pn.conv), W)


def test_noalloc_step_rejects_too_many_rows():
    """Rows whose workspace exceeds the library's array are refused before
    anything is enqueued, and the pools stay untouched."""
    s = wl.FULL_HEADS
    L = Layer(s, wl.layer_weights(np.random.default_rng(1), s))
    B = 4097
    assert gdn.gdn_decode_workspace_bytes(L.geom, B) > (1 << 20)
    rec = torch.zeros(1, s.num_v_heads, s.head_k_dim, s.head_v_dim, device="cuda")
    conv = torch.zeros(1, s.conv_kernel, s.channels, device="cuda", dtype=torch.bfloat16)
    pool = gdn.StatePool(L.geom, rec, conv)
    bf = torch.bfloat16
    with pytest.raises(gdn.GdnError, match="workspace"):
        gdn.gdn_decode_step_noalloc(
            L.geom, L.w, pool, torch.full((B,), -1, device="cuda", dtype=torch.int32),
            torch.zeros(B, s.channels, device="cuda", dtype=bf),
            torch.zeros(B, s.num_v_heads, s.head_v_dim, device="cuda", dtype=bf),
            torch.zeros(B, s.num_v_heads, device="cuda", dtype=bf),
            torch.zeros(B, s.num_v_heads, device="cuda", dtype=bf),
            torch.empty(B, s.num_v_heads, s.head_v_dim, device="cuda", dtype=bf))
