"""gdn_check_slots on the GPU: the device-side check of a device-resident slot
index against the rule the host check applies (negative = padding, else in
[0, num_slots), no slot named twice), on random and edge-case indexes, eager
and replayed from a HIP graph with the index rewritten in place."""
import numpy as np
import pytest
import torch

import linear_attention_causal_amd as gdn

pytestmark = pytest.mark.gpu
INT_MAX = 2 ** 31 - 1


def expected(slots, P):
    """(status, first offending row) by the rule, on the host."""
    seen = set()
    for b, s in enumerate(slots):
        if s >= P or (s >= 0 and s in seen):
            return gdn._abi.GDN_E_SLOT, b
        if s >= 0:
            seen.add(s)
    return gdn._abi.GDN_OK, INT_MAX


def run(slots, P):
    res = torch.full((2,), 123, device="cuda", dtype=torch.int32)
    sl = torch.from_numpy(np.asarray(slots, np.int32)).cuda()
    gdn.gdn_check_slots(sl, P, res)
    torch.cuda.synchronize()
    return tuple(res.cpu().tolist())


def test_check_slots_cases():
    rng = np.random.default_rng(3)
    cases = [([], 4), ([0], 4), ([-1, -1, -1], 4), ([3, 1, 2, 0], 4), ([3, 1, 3], 4),
             ([0, 4], 4), ([-1, 7, -3, 2], 8), ([5, 5], 8), ([1, -1, 1], 8)]
    for B, P in [(16, 64), (256, 320), (257, 320), (600, 4096), (3000, 8192)]:
        ok = rng.choice(P, B, replace=False).astype(np.int32)
        ok[rng.random(B) < 0.1] = -1
        cases.append((ok.tolist(), P))
        dup = ok.copy()
        i, j = sorted(rng.choice(B, 2, replace=False))
        dup[i] = 5
        dup[j] = 5                        # j repeats row i's slot
        cases.append((dup.tolist(), P))
        far = ok.copy()
        far[rng.integers(B)] = P + 3      # out of range
        cases.append((far.tolist(), P))
        both = dup.copy()
        both[min(i, j) // 2] = P          # an earlier range error
        cases.append((both.tolist(), P))
    for slots, P in cases:
        got = run(slots, P)
        exp = expected(slots, P)
        assert got == exp, (len(slots), P, got, exp)
    print(f"  {len(cases)} slot indexes checked", flush=True)


def test_check_slots_in_a_graph():
    """Captured once with the check ahead of nothing else; replays see the
    index rewritten in place and report each state anew."""
    P, B = 64, 16
    sl = torch.arange(B, device="cuda", dtype=torch.int32)
    res = torch.zeros(2, device="cuda", dtype=torch.int32)
    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            gdn.gdn_check_slots(sl, P, res, stream=side)
    stream.wait_stream(side)
    rng = np.random.default_rng(9)
    for rep in range(6):
        v = rng.choice(P, B, replace=False).astype(np.int32)
        if rep % 2:
            v[B - 1] = v[2]
        sl.copy_(torch.from_numpy(v))
        graph.replay()
        torch.cuda.synchronize()
        assert tuple(res.cpu().tolist()) == expected(v.tolist(), P), rep
