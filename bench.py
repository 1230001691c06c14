"""Benchmark of the Gated DeltaNet layer core on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Headline (`value`): batched decode at one rank's share of the heads, B = 16
rows, Hk = 8, Hv = 16, dk = dv = 128, bf16 activations, f32 state, 64-slot
pool.  One step = gdn_decode_step (conv update, state update and gated
RMSNorm in one launch) for the 16 rows of one layer.  Steps rotate over 16 layer replicas (pools, weights and inputs) so
that every step streams its state from HBM rather than from the 256 MB
last-level cache, as consecutive layers of a model do.

Also reported on the same JSON line:
  roofline      the fused decode kernel: algorithmic bytes per launch / its
                mean duration from HIP events on the launch stream, vs 8 TB/s;
  prefill       4096-token single-sequence prefill (Hk=8, Hv=16) and the
                8-sequence packed varlen prefill (Hk=16, Hv=32): tokens/s and
                algorithmic MFMA fraction;
  block         one decode token per row through the whole block (input
                projections, the layer, out_proj; hidden 2048) at B = 16
                rank-local and B = 256 full-head, with the library GEMM timed
                beside the projection kernel;
  serving       B = 256 rows through 48 layers (Hk=16, Hv=32, 320-slot pools)
                with a retire + compaction event every 16 steps;
  cpu_baseline  the f64 oracle on the host cores, on a bounded sample of the
                headline workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GDN decode tokens/s + % HBM peak; chunked prefill tokens/s + % MFMA"
HBM_PEAK = 8.0e12            # bytes/s
BF16_PEAK = 2.5e15           # dense MFMA flop/s
F32_MFMA_PEAK = 157.3e12     # dense f32 MFMA flop/s
PREFILL_FLOP_PER_TOKEN_HEAD = 180_224   # chunk contractions at d = 128, L = 64
GRAPH_PASSES = 4             # passes over the layer replicas per captured decode graph


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--replicas", type=int, default=16)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="headline decode only (for profiler runs)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--calibration-copy", action="store_true",
                    help="also run a plain 512 MiB device copy kernel (the reference "
                         "for scaling the HBM byte counters of a profiler run)")
    ap.add_argument("--calibration-gemm", action="store_true",
                    help="also run a bf16 8192^3 library GEMM (a reference reading for "
                         "the MFMA-busy counters of a profiler run)")
    ap.add_argument("--block-only", action="store_true",
                    help="only the decode-block legs (projections + layer)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="run only the two prefill workloads and print their figures "
                         "(for profiler runs of the prefill kernels)")
    return ap.parse_args()


# ------------------------------------------------------------------ helpers


def _t(x, dtype):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(dtype).contiguous()


class DecodeLayer:
    """Device copies of one layer's weights, pool and one step of inputs."""

    def __init__(self, gdn, geom, data, act):
        import torch
        self.keep = dict(conv_w=_t(data["weights"]["conv_w"], act),
                         A_log=_t(data["weights"]["A_log"], torch.float32),
                         dt_bias=_t(data["weights"]["dt_bias"], torch.float32),
                         norm_w=_t(data["weights"]["norm_w"], torch.float32))
        self.w = gdn.LayerWeights(geom, **{"conv_weight": self.keep["conv_w"],
                                           "A_log": self.keep["A_log"],
                                           "dt_bias": self.keep["dt_bias"],
                                           "norm_weight": self.keep["norm_w"]})
        self.rec = _t(data["rec"], torch.float32)
        self.conv = _t(data["conv"], act)
        self.pool = gdn.StatePool(geom, self.rec, self.conv)
        self.slot = _t(data["slot_idx"], torch.int32)
        self.x = _t(data["x"], act)
        self.z = _t(data["z"], act)
        self.a = _t(data["a"], act)
        self.b = _t(data["b"], act)


def step_bytes(geom, B, act_bytes):
    """Algorithmic bytes of one decode step (conv update + decode) per layer:
    state read + write, conv window (K-1 columns read, K written), the token's
    fused input, z, a, b and y."""
    C, Hv, dk, dv, K = (geom.channels, geom.num_v_heads, geom.head_k_dim, geom.head_v_dim,
                        geom.conv_kernel)
    return B * (8 * Hv * dk * dv + (2 * K - 1) * C * act_bytes + C * act_bytes
                + 2 * Hv * dv * act_bytes + 2 * Hv * act_bytes)


# ------------------------------------------------------------------ decode


def bench_decode(args):
    """The headline step, replayed from a HIP graph (one graph = one pass over
    the layer replicas), as the pages' serving path replays captured decode
    steps.  An eager (one Python launch per step) figure is reported beside it."""
    import numpy as np
    import torch

    import linear_attention_causal_amd as gdn
    import workloads as wl

    work = wl.decode_batch(seed=0)
    s = work.shape
    geom = gdn.Geometry(s.num_k_heads, s.num_v_heads, s.head_k_dim, s.head_v_dim,
                        s.conv_kernel, s.act)
    act = torch.bfloat16
    B = len(work.data["slot_idx"])
    R = args.replicas
    layers = [DecodeLayer(gdn, geom, work.data, act) for _ in range(R)]
    y = torch.empty(B, geom.num_v_heads, geom.head_v_dim, device="cuda", dtype=act)
    ws = gdn.decode_workspace(geom, B)

    def step(i, stream):
        L = layers[i % R]
        gdn.gdn_decode_step(geom, L.w, L.pool, L.slot, L.x, L.z, L.a, L.b, y, ws, stream=stream)

    stream = torch.cuda.current_stream()
    for i in range(args.warmup):
        step(i, stream)
    torch.cuda.synchronize()
    # eager: one Python-side launch per step
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, stream)
    torch.cuda.synchronize()
    eager_dt = time.perf_counter() - t0

    # graph: G = GRAPH_PASSES * R steps (passes over the replicas) captured
    # once, replayed; more steps per graph spread the replay's own launch cost
    G = GRAPH_PASSES * R
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            for i in range(G):
                step(i, side)
    stream.wait_stream(side)
    for _ in range(max(1, args.warmup // G)):
        graph.replay()
    torch.cuda.synchronize()
    reps = max(1, args.steps // G)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    t0 = time.perf_counter()
    for k in range(reps):
        evs[k][0].record(stream)
        graph.replay()
        evs[k][1].record(stream)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    nsteps = reps * G
    launch_ms = float(np.mean([a.elapsed_time(b) for a, b in evs])) / G
    per_launch = step_bytes(geom, B, 2)
    achieved = per_launch / (launch_ms * 1e-3)
    rec = recorded_traffic()
    return dict(
        tokens_per_s=B * nsteps / dt, ms_per_step=dt * 1e3 / nsteps, steps=nsteps, B=B,
        workload=work.name, geom=geom,
        eager={"tokens_per_s": B * args.steps / eager_dt,
               "ms_per_step": eager_dt * 1e3 / args.steps},
        roofline={"bound": "hbm", "achieved": achieved / 1e9, "peak": HBM_PEAK / 1e9,
                  "unit": "GB/s", "frac": achieved / HBM_PEAK,
                  "traffic": rec["hbm_bytes_per_launch"] if rec else None,
                  "traffic_unit": "HBM bytes per launch (scaled FETCH_SIZE + WRITE_SIZE)",
                  "kernel": "gdn::decode_head_kernel<__bf16, 128, 4, 1>",
                  "bytes_per_launch": per_launch, "mean_launch_us": launch_ms * 1e3,
                  "timing": f"HIP events around graph replays of {G} back-to-back launches "
                            f"({GRAPH_PASSES} passes over {R} replicas)"},
        step_hbm_frac=per_launch / (dt / nsteps) / HBM_PEAK)


TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "decode_step_b16_hk8_hv16_d128_traffic.md")
TRAFFIC_SOURCES = ("linear_attention_causal_amd/csrc/decode.hip",
                   "linear_attention_causal_amd/csrc/gdn_device.hpp")
MFMA_RECORD = os.path.join(ROOT, "profiles", "prefill_t4096_varlen8_d128.md")
MFMA_SOURCES = ("linear_attention_causal_amd/csrc/prefill.hip",
                "linear_attention_causal_amd/csrc/gdn_device.hpp")


def kernel_source_digest(sources=TRAFFIC_SOURCES):
    import hashlib
    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def read_record(path, sources):
    """The `record:` line of a committed profiler summary, or None when there is
    none or the kernel sources have changed since the counters were taken."""
    try:
        with open(path) as f:
            text = f.read()
    except OSError:
        return None
    rec = None
    for ln in text.splitlines():
        if ln.startswith("record: "):
            rec = json.loads(ln[len("record: "):])
    if not rec or rec.get("source_sha256") != kernel_source_digest(sources):
        return None
    return rec


def recorded_traffic():
    """HBM bytes per decode launch from the committed counter record (FETCH_SIZE
    and WRITE_SIZE passes, each scaled by the same counter's reading on a plain
    copy of known size)."""
    return read_record(TRAFFIC_RECORD, TRAFFIC_SOURCES)


def recorded_mfma_util(workload):
    """MFMA-pipe utilisation (percent, kernel-time weighted over a prefill call)
    from the committed counter record, or None."""
    rec = read_record(MFMA_RECORD, MFMA_SOURCES)
    return rec["mfma_pipe_util_pct"].get(workload) if rec else None


def calibration_copy(nbytes=512 << 20, reps=4):
    """A plain elementwise copy (read nbytes, write nbytes) run a few times; its
    counter readings calibrate FETCH_SIZE / WRITE_SIZE."""
    import torch
    src = torch.ones(nbytes // 4, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    log(f"[bench] calibration copy: {nbytes} bytes read + {nbytes} written per launch, {reps} launches")


def calibration_gemm(n=8192, reps=4):
    """A bf16 n^3 matmul through the library GEMM: a kernel that keeps the MFMA
    pipes busy, to read the MFMA-busy counters against."""
    import torch
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    for _ in range(reps):
        torch.matmul(a, b)
    torch.cuda.synchronize()
    log(f"[bench] calibration gemm: bf16 {n}^3, {reps} launches")


# ------------------------------------------------------------------ prefill


def bench_prefill(work, iters, replicas):
    import numpy as np
    import torch

    import linear_attention_causal_amd as gdn

    s, d = work.shape, work.data
    geom = gdn.Geometry(s.num_k_heads, s.num_v_heads, s.head_k_dim, s.head_v_dim,
                        s.conv_kernel, s.act)
    act = torch.bfloat16
    cu = d["cu_seqlens"]
    T, N = int(cu[-1]), len(cu) - 1
    w = dict(conv_w=_t(d["weights"]["conv_w"], act), A_log=_t(d["weights"]["A_log"], torch.float32),
             dt_bias=_t(d["weights"]["dt_bias"], torch.float32),
             norm_w=_t(d["weights"]["norm_w"], torch.float32))
    lw = gdn.LayerWeights(geom, w["conv_w"], w["A_log"], w["dt_bias"], w["norm_w"])
    rec = _t(d["rec"], torch.float32)
    conv = _t(d["conv"], act)
    pool = gdn.StatePool(geom, rec, conv)
    inputs = []
    x0, z0, a0, b0 = (_t(d[k], act) for k in ("x", "z", "a", "b"))
    for r in range(replicas):
        inputs.append((x0.clone(), z0.clone(), a0.clone(), b0.clone()))
    del x0, z0, a0, b0
    cu_d = _t(cu, torch.int32)
    slots = _t(d["slot_idx"], torch.int32)
    has_init = _t(d["has_init"], torch.uint8)
    y = torch.empty(T, geom.num_v_heads, geom.head_v_dim, device="cuda", dtype=act)
    scratch = torch.empty(gdn.gdn_prefill_scratch_bytes(geom, T, N), device="cuda",
                          dtype=torch.uint8)
    stream = torch.cuda.current_stream()

    def call(i):
        x, z, a, b = inputs[i % replicas]
        gdn.gdn_prefill_chunked(geom, lw, pool, cu, cu_d, slots, x, z, a, b, y, scratch,
                                has_init=has_init, stream=stream)

    call(0)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(iters)]
    for i in range(iters):
        ev[i][0].record(stream)
        call(i + 1)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
    flops = PREFILL_FLOP_PER_TOKEN_HEAD * T * geom.num_v_heads * (geom.head_k_dim / 128) ** 2
    return {"workload": work.name, "tokens": T, "sequences": N, "ms_per_call": ms,
            "tokens_per_s": T / (ms * 1e-3),
            "algorithmic_tflops": flops / (ms * 1e-3) / 1e12,
            "mfma_frac_of_bf16_peak": flops / (ms * 1e-3) / BF16_PEAK,
            "mfma_frac_of_f32_peak": flops / (ms * 1e-3) / F32_MFMA_PEAK,
            "mfma_pipe_util_pct": recorded_mfma_util(work.name),
            "mfma_pipe_util_source": "rocprofv3 MfmaUtil, kernel-time weighted over the call "
                                     "(committed prefill profile record; null once the "
                                     "kernels change)",
            "mfma_dtype": "bf16 x3 (hi/lo split operands, f32 accumulate)", "kernels": 4}


# ------------------------------------------------------------------ block


def _graph_us(fn, R, warm=2, reps=20):
    """Mean device time (us) of one of R back-to-back calls fn(r), captured
    once in a HIP graph and replayed, from HIP events on the replay stream."""
    import numpy as np
    import torch

    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        for r in range(R):          # eager pass first: library workspaces allocated outside
            fn(r, side)
        with torch.cuda.graph(graph, stream=side):
            for r in range(R):
                fn(r, side)
    stream.wait_stream(side)
    for _ in range(warm):
        graph.replay()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for a, b in evs:
        a.record(stream)
        graph.replay()
        b.record(stream)
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in evs])) * 1e3 / R


def bench_block(B, shape, P, replicas):
    """One decode token per row through the whole block: the four input
    projections (one gdn_linear launch), gdn_decode_step, and out_proj (one
    gdn_linear launch), on `replicas` rotating copies of the weights and pools
    so that every block streams its weights and state from HBM.  Each part is
    also timed on its own, and the five projections are timed through the
    library GEMM (torch.mm on pre-transposed weights) for comparison."""
    import torch

    import linear_attention_causal_amd as gdn
    import workloads as wl

    work = wl.decode_block(seed=0, B=B, P=P, s=shape)
    s, d = work.shape, work.data
    geom = gdn.Geometry(s.num_k_heads, s.num_v_heads, s.head_k_dim, s.head_v_dim,
                        s.conv_kernel, s.act)
    bf = torch.bfloat16
    H = d["hidden"].shape[1]
    C, Hv, vd = s.channels, s.num_v_heads, s.num_v_heads * s.head_v_dim
    wd = dict(conv_w=_t(d["weights"]["conv_w"], bf),
              A_log=_t(d["weights"]["A_log"], torch.float32),
              dt_bias=_t(d["weights"]["dt_bias"], torch.float32),
              norm_w=_t(d["weights"]["norm_w"], torch.float32))
    lw = gdn.LayerWeights(geom, wd["conv_w"], wd["A_log"], wd["dt_bias"], wd["norm_w"])
    proj0 = {k: _t(v, bf) for k, v in d["proj"].items()}
    rec0, conv0 = _t(d["rec"], torch.float32), _t(d["conv"], bf)
    reps = []
    for r in range(replicas):
        rec, conv = rec0.clone(), conv0.clone()
        reps.append(dict(p={k: v.clone() for k, v in proj0.items()}, rec=rec, conv=conv,
                         pool=gdn.StatePool(geom, rec, conv), h=_t(d["hidden"], bf)))
    del proj0, rec0, conv0
    slot = _t(d["slot_idx"], torch.int32)
    qkv = torch.empty(B, C, device="cuda", dtype=bf)
    z = torch.empty(B, vd, device="cuda", dtype=bf)
    bb = torch.empty(B, Hv, device="cuda", dtype=bf)
    aa = torch.empty(B, Hv, device="cuda", dtype=bf)
    y = torch.empty(B, vd, device="cuda", dtype=bf)
    out = torch.empty(B, H, device="cuda", dtype=bf)
    ws = gdn.decode_workspace(geom, B)

    def in_proj(r, st):
        R = reps[r]
        gdn.gdn_linear(R["h"], [(R["p"]["qkv"], qkv), (R["p"]["z"], z), (R["p"]["b"], bb),
                                (R["p"]["a"], aa)], stream=st)

    def core(r, st):
        gdn.gdn_decode_step(geom, lw, reps[r]["pool"], slot, qkv, z, aa, bb, y, ws, stream=st)

    def out_proj(r, st):
        gdn.gdn_linear(y, [(reps[r]["p"]["out"], out)], stream=st)

    def block(r, st):
        in_proj(r, st)
        core(r, st)
        out_proj(r, st)

    R = replicas
    t_block = _graph_us(block, R)
    t_in = _graph_us(in_proj, R)
    t_core = _graph_us(core, R)
    t_out = _graph_us(out_proj, R)
    # library GEMM on the same weights, pre-transposed to [in][out] (no transposed views)
    lib_w = [{k: v.t().contiguous() for k, v in R_["p"].items()} for R_ in reps]

    def lib_in(r, st):
        h = reps[r]["h"]
        for k, o in (("qkv", qkv), ("z", z), ("b", bb), ("a", aa)):
            torch.mm(h, lib_w[r][k], out=o)

    def lib_out(r, st):
        torch.mm(y, lib_w[r]["out"], out=out)

    t_lib_in = _graph_us(lib_in, R)
    t_lib_out = _graph_us(lib_out, R)
    n_in = C + vd + 2 * Hv
    in_bytes = 2 * (n_in * H + B * H + B * n_in)
    out_bytes = 2 * (H * vd + B * vd + B * H)
    core_bytes = step_bytes(geom, B, 2)
    total = in_bytes + core_bytes + out_bytes
    flops = 2 * B * H * (n_in + vd)
    return {"workload": work.name, "rows": B, "hidden": H, "num_k_heads": s.num_k_heads,
            "num_v_heads": Hv, "head_dim": s.head_k_dim, "launches": 3,
            "us_per_block": t_block, "tokens_per_s": B / (t_block * 1e-6),
            "block_bytes": total, "block_hbm_frac": total / (t_block * 1e-6) / HBM_PEAK,
            "in_proj_us": t_in, "in_proj_hbm_frac": in_bytes / (t_in * 1e-6) / HBM_PEAK,
            "decode_step_us": t_core,
            "out_proj_us": t_out, "out_proj_hbm_frac": out_bytes / (t_out * 1e-6) / HBM_PEAK,
            "projection_tflops": flops / ((t_in + t_out) * 1e-6) / 1e12,
            "library_in_proj_us": t_lib_in, "library_out_proj_us": t_lib_out,
            "library": "torch.mm (hipBLASLt), four input launches + one output launch",
            "timing": f"HIP events around graph replays of {R} back-to-back blocks on "
                      f"{R} weight/pool replicas"}


# ------------------------------------------------------------------ serving


def bench_serving(steps=32, layers=48, B=256, P=320):
    """B rows through `layers` layers per step; after every 16 steps a seeded
    half of the rows retire, survivors are compacted across all layers and
    new rows are admitted (zero state).  Pools and inputs are drawn on the
    device from a seeded generator."""
    import numpy as np
    import torch

    import linear_attention_causal_amd as gdn
    import workloads as wl

    s = wl.FULL_HEADS
    geom = gdn.Geometry(s.num_k_heads, s.num_v_heads, s.head_k_dim, s.head_v_dim,
                        s.conv_kernel, s.act)
    act = torch.bfloat16
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0)
    rng = np.random.default_rng(0)
    C = geom.channels
    Ls = []
    for _ in range(layers):
        w = wl.layer_weights(rng, s)
        keep = (_t(w["conv_w"], act), _t(w["A_log"], torch.float32),
                _t(w["dt_bias"], torch.float32), _t(w["norm_w"], torch.float32))
        rec = torch.randn(P, s.num_v_heads, s.head_k_dim, s.head_v_dim, device="cuda",
                          generator=gen) * 0.1
        conv = (torch.randn(P, s.conv_kernel, C, device="cuda", generator=gen) * 0.1).to(act)
        Ls.append(dict(keep=keep, w=gdn.LayerWeights(geom, *keep), rec=rec, conv=conv,
                       pool=gdn.StatePool(geom, rec, conv)))
    live = np.sort(rng.choice(P, B, replace=False)).astype(np.int32)
    x = (torch.randn(B, C, device="cuda", generator=gen)).to(act)
    z = torch.randn(B, s.num_v_heads, s.head_v_dim, device="cuda", generator=gen).to(act)
    a = torch.randn(B, s.num_v_heads, device="cuda", generator=gen).to(act)
    b = torch.randn(B, s.num_v_heads, device="cuda", generator=gen).to(act)
    y = torch.empty(B, s.num_v_heads, s.head_v_dim, device="cuda", dtype=act)
    stream = torch.cuda.current_stream()
    pools = [L["pool"] for L in Ls]
    compact_ms = []
    # device-resident slot index: the captured step reads it, a retire event
    # rewrites it in place
    slot_d = _t(live, torch.int32)
    ws = gdn.decode_workspace(geom, B)

    def layer_pass(st):
        for L in Ls:
            gdn.gdn_decode_step(geom, L["w"], L["pool"], slot_d, x, z, a, b, y, ws, stream=st)

    graph = None

    def run(nsteps, live, use_graph):
        for t in range(nsteps):
            if t > 0 and t % 16 == 0:
                keep, new_slots, src, dst = wl.retire_plan(rng, live, P)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                if src.size:
                    gdn.gdn_state_compact(geom, pools, src, dst, _t(src, torch.int32),
                                          _t(dst, torch.int32), stream=stream)
                e1.record(stream)
                compact_ms.append((e0, e1, int(src.size)))
                admitted = np.arange(len(new_slots), len(new_slots) + (len(live) - len(new_slots)),
                                     dtype=np.int32)
                live = np.concatenate([new_slots, admitted]).astype(np.int32)
                slot_d.copy_(torch.from_numpy(live))
            if use_graph:
                graph.replay()
            else:
                layer_pass(stream)
        return live

    live = run(2, live, False)
    torch.cuda.synchronize()
    compact_ms.clear()
    t0 = time.perf_counter()
    live = run(steps, live, False)
    torch.cuda.synchronize()
    eager_dt = time.perf_counter() - t0
    compact_ms.clear()
    # one HIP graph per step: the 48 layer launches captured once
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            layer_pass(side)
    stream.wait_stream(side)
    graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run(steps, live, True)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    cms = [a_.elapsed_time(b_) for a_, b_, _ in compact_ms]
    moved = [n for _, _, n in compact_ms]
    per_step = layers * step_bytes(geom, B, 2)
    return {"workload": f"decode_b{B}_hk16_hv32_d128_p{P}_x{layers}layers",
            "launch": "HIP graph of the 48 layer launches per step, replayed",
            "tokens_per_s": B * steps / dt, "ms_per_step": dt * 1e3 / steps,
            "hbm_frac_algorithmic": per_step * steps / dt / HBM_PEAK,
            "eager_tokens_per_s": B * steps / eager_dt,
            "compaction_events": len(cms), "compaction_ms": cms, "compaction_pairs": moved,
            "steps": steps}


# ------------------------------------------------------------------ CPU oracle


def cpu_baseline(seconds):
    """The f64 oracle (as it stands) on the host cores: decode steps of the
    headline workload (16 rows, Hk=8, Hv=16, d=128), repeated until about
    `seconds` of wall time has passed."""
    import numpy as np

    import oracle
    import workloads as wl

    work = wl.decode_batch(seed=0)
    s, d = work.shape, work.data
    og = oracle.Geometry(s.num_k_heads, s.num_v_heads, s.head_k_dim, s.head_v_dim,
                         s.conv_kernel)
    ow = oracle.Weights(d["weights"]["conv_w"], d["weights"]["A_log"], d["weights"]["dt_bias"],
                        d["weights"]["norm_w"])
    S, W = d["rec"].astype(np.float64), d["conv"].astype(np.float64)
    B = len(d["slot_idx"])
    def run(threads, budget):
        n = 0
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < budget:
            oracle.pool_run(og, ow, S, W, np.arange(B + 1), d["slot_idx"], d["x"], d["z"],
                            d["a"], d["b"], nthreads=threads)
            n += 1
        return n, time.perf_counter() - t0

    threads = oracle.default_threads()
    n, dt = run(threads, seconds)
    n1, dt1 = run(1, max(2.0, seconds / 4))
    return {"value": B * n / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "single_thread_value": B * n1 / dt1,
            "sample": f"{n} decode steps of the headline workload (16 rows x 16 V-heads, "
                      f"d=128) in {dt:.1f} s, f64, one thread per (row, V-head) unit; "
                      f"single thread: {n1} steps in {dt1:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch

    import linear_attention_causal_amd as gdn

    gdn.library()
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    if args.prefill_only:
        import workloads as wl
        if args.calibration_gemm:
            calibration_gemm()
        out = [bench_prefill(wl.prefill_single(seed=0), iters=10, replicas=6)]
        torch.cuda.empty_cache()
        out.append(bench_prefill(wl.prefill_varlen(seed=0), iters=5, replicas=1))
        print(json.dumps({"prefill": out}), flush=True)
        return
    if args.block_only:
        import workloads as wl
        out = [bench_block(16, wl.RANK_LOCAL, 64, args.replicas)]
        torch.cuda.empty_cache()
        out.append(bench_block(256, wl.FULL_HEADS, 320, 4))
        print(json.dumps({"block": out}), flush=True)
        return
    log("[bench] decode headline")
    dec = bench_decode(args)
    if args.calibration_copy:
        calibration_copy()
    if args.calibration_gemm:
        calibration_gemm()
    line = {
        "metric": METRIC, "value": dec["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": dec["steps"], "warmup": args.warmup, "ms_per_step": dec["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": dec["workload"], "rows": dec["B"], "num_k_heads": 8,
                   "num_v_heads": 16, "head_dim": 128, "conv_kernel": 4, "pool_slots": 64,
                   "activations": "bf16", "state": "f32",
                   "cold_cache": f"{args.replicas} rotating layer replicas",
                   "launch": "HIP graph replay"},
        "eager": dec["eager"],
        "step_hbm_frac_algorithmic": dec["step_hbm_frac"],
        "roofline": dec["roofline"],
    }
    if not args.no_extras:
        import workloads as wl
        log("[bench] prefill t4096")
        pre = [bench_prefill(wl.prefill_single(seed=0), iters=10, replicas=6)]
        torch.cuda.empty_cache()
        log("[bench] prefill varlen8")
        pre.append(bench_prefill(wl.prefill_varlen(seed=0), iters=5, replicas=1))
        torch.cuda.empty_cache()
        line["prefill"] = pre
        log("[bench] decode block b16")
        line["block"] = [bench_block(16, wl.RANK_LOCAL, 64, args.replicas)]
        torch.cuda.empty_cache()
        log("[bench] decode block b256")
        line["block"].append(bench_block(256, wl.FULL_HEADS, 320, 4))
        torch.cuda.empty_cache()
        log("[bench] serving 48 layers")
        line["serving"] = bench_serving()
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline")
        line["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
