"""Benchmark of the Gated DeltaNet layer core on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Headline (`value`): batched decode at one rank's share of the heads, B = 16
rows, Hk = 8, Hv = 16, dk = dv = 128, bf16 activations, f32 state, 64-slot
pool.  One step = gdn_decode_step (conv update, state update and gated
RMSNorm in one launch) for the 16 rows of one layer.  Steps rotate over 16
layer replicas (pools, weights and inputs) so that every step streams its
state from HBM rather than from the 256 MB last-level cache, as consecutive
layers of a model do.  Exactly K steps run in the timed region, replayed
from HIP graphs captured beforehand (the captured-graph decode of serving).

Also reported on the same JSON line:
  roofline      the fused decode kernel: algorithmic bytes per launch / its
                mean duration from HIP events on the launch stream over a
                1024-launch graph replay, vs 8 TB/s; HBM traffic per launch
                from the committed counter record;
  prefill       the 4096-token single-sequence prefill (Hk=8, Hv=16) and the
                8-sequence packed varlen prefill (Hk=16, Hv=32): median call
                time over 100 calls, tokens/s, an HBM roofline object (the
                whole call is HBM-bound by its algorithm) and the MFMA
                figures (algorithmic fraction of the bf16 peak; MFMA-pipe
                utilisation from the committed counter record);
  serving       B = 256 rows through 48 layers (Hk=16, Hv=32, 320-slot
                pools), 64 steps with a retire + compaction + admission
                event after steps 16, 32 and 48; roofline of its layer launch;
  block         one decode token per row through the whole block (input
                projections, the layer, out_proj; hidden 2048) at B = 16
                rank-local and B = 256 full-head, with the library GEMM timed
                beside the projection kernel;
  cpu_baseline  the f64 oracle on the host cores for the headline workload,
                and `cpu_baselines` for every workload, each at one thread
                and at all the threads the oracle uses, on bounded samples.
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
PREFILL_FLOP_PER_TOKEN_HEAD = 180_224   # chunk contractions at d = 128, L = 64
ROOFLINE_GRAPH = 1024        # launches per graph for the roofline's mean launch time
LEGS = ("decode", "prefill", "block", "serving")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--replicas", type=int, default=16)
    ap.add_argument("--legs", default=",".join(LEGS),
                    help="comma-separated subset of " + ",".join(LEGS) +
                         " (the headline decode always runs unless --prefill-only)")
    ap.add_argument("--prefill-iters", type=int, default=100)
    ap.add_argument("--serving-steps", type=int, default=64)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="headline decode only (for profiler runs)")
    ap.add_argument("--cpu-seconds", type=float, default=2.0,
                    help="wall-time budget of each oracle sample loop")
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


def geometry(gdn, s):
    return gdn.Geometry(s.num_k_heads, s.num_v_heads, s.head_k_dim, s.head_v_dim,
                        s.conv_kernel, s.act)


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


def prefill_bytes(geom, T, N, act_bytes):
    """Algorithmic bytes of one prefill call: per token the fused input (C),
    z and y (Hv dv each) and a, b (Hv each); per sequence the recurrent
    state read and written and the conv window (K-1 columns read, K written)."""
    C, Hv, dk, dv, K = (geom.channels, geom.num_v_heads, geom.head_k_dim, geom.head_v_dim,
                        geom.conv_kernel)
    per_token = (C + 2 * Hv * dv + 2 * Hv) * act_bytes
    per_seq = 8 * Hv * dk * dv + (2 * K - 1) * C * act_bytes
    return T * per_token + N * per_seq


def capture(fn):
    """Capture fn(stream) on a side stream into a HIP graph (nothing runs)."""
    import torch
    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            fn(side)
    stream.wait_stream(side)
    return graph


# ------------------------------------------------------------------ records


TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "decode_step_b16_hk8_hv16_d128_traffic.md")
SERVING_RECORD = os.path.join(ROOT, "profiles", "decode_step_b256_hk16_hv32_d128_traffic.md")
DECODE_SOURCES = ("linear_attention_causal_amd/csrc/decode.hip",
                  "linear_attention_causal_amd/csrc/gdn_device.hpp")
MFMA_RECORD = os.path.join(ROOT, "profiles", "prefill_t4096_varlen8_d128.md")
PREFILL_TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "prefill_t4096_varlen8_d128_traffic.md")
PREFILL_SOURCES = ("linear_attention_causal_amd/csrc/prefill.hip",
                   "linear_attention_causal_amd/csrc/gdn_device.hpp")


def kernel_source_digest(sources):
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


def recorded_traffic(path, key="hbm_bytes_per_launch"):
    """HBM bytes per launch from a committed counter record (FETCH_SIZE and
    WRITE_SIZE passes, each scaled by the same counter's reading on a plain
    copy of known size), or None."""
    rec = read_record(path, DECODE_SOURCES)
    return rec.get(key) if rec else None


def recorded_prefill(workload):
    """(MFMA-pipe utilisation percent, HBM bytes per call) of a prefill workload
    from the committed counter records, each None when absent or stale."""
    m = read_record(MFMA_RECORD, PREFILL_SOURCES)
    t = read_record(PREFILL_TRAFFIC_RECORD, PREFILL_SOURCES)
    return (m["mfma_pipe_util_pct"].get(workload) if m else None,
            t["hbm_bytes_per_call"].get(workload) if t else None)


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


# ------------------------------------------------------------------ decode


def bench_decode(args):
    """The headline step.  Exactly args.steps launches run in the timed
    region, replayed from HIP graphs (one of min(K, 1024) launches replayed
    K // 1024 times, plus one of the remainder), bracketed by a device
    synchronisation on both sides; the wall time between gives `value`.
    The roofline's mean launch duration comes from HIP events on the replay
    stream around separate replays of a 1024-launch graph.  An eager (one
    Python launch per step) figure is reported beside it."""
    import numpy as np
    import torch

    import linear_attention_causal_amd as gdn
    import workloads as wl

    work = wl.decode_batch(seed=0)
    s = work.shape
    geom = geometry(gdn, s)
    act = torch.bfloat16
    B = len(work.data["slot_idx"])
    R = args.replicas
    K = max(1, args.steps)
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
    # eager: one Python-side launch per step (not the headline)
    n_eager = max(K, 64)
    t0 = time.perf_counter()
    for i in range(n_eager):
        step(i, stream)
    torch.cuda.synchronize()
    eager_dt = time.perf_counter() - t0

    # timed region: exactly K launches from captured graphs
    G = min(K, ROOFLINE_GRAPH)
    full, rem = divmod(K, G)
    g_full = capture(lambda st: [step(i, st) for i in range(G)])
    g_rem = capture(lambda st: [step(full * G + i, st) for i in range(rem)]) if rem else None
    g_full.replay()                      # untimed: first replay uploads the graph
    if g_rem is not None:
        g_rem.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(full):
        g_full.replay()
    if g_rem is not None:
        g_rem.replay()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0

    # roofline: mean launch duration over replays of a 1024-launch graph
    g_roof = capture(lambda st: [step(i, st) for i in range(ROOFLINE_GRAPH)])
    g_roof.replay()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(4)]
    for e0, e1 in evs:
        e0.record(stream)
        g_roof.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    launch_ms = float(np.mean([a.elapsed_time(b) for a, b in evs])) / ROOFLINE_GRAPH
    per_launch = step_bytes(geom, B, 2)
    achieved = per_launch / (launch_ms * 1e-3)
    return dict(
        tokens_per_s=B * K / dt, ms_per_step=dt * 1e3 / K, steps=K, B=B,
        workload=work.name, geom=geom,
        eager={"tokens_per_s": B * n_eager / eager_dt, "ms_per_step": eager_dt * 1e3 / n_eager,
               "steps": n_eager},
        timed_region={"launches": K, "graphs": f"{full} x {G} launches" +
                      (f" + 1 x {rem}" if rem else ""), "wall_s": dt},
        roofline={"bound": "hbm", "achieved": achieved / 1e9, "peak": HBM_PEAK / 1e9,
                  "unit": "GB/s", "frac": achieved / HBM_PEAK,
                  "traffic": recorded_traffic(TRAFFIC_RECORD),
                  "traffic_unit": "HBM bytes per launch (scaled FETCH_SIZE + WRITE_SIZE)",
                  "kernel": "gdn::decode_head_kernel<__bf16, 128, 4>",
                  "bytes_per_launch": per_launch, "mean_launch_us": launch_ms * 1e3,
                  "timing": f"HIP events on the launch stream around 4 replays of a graph of "
                            f"{ROOFLINE_GRAPH} back-to-back launches ({ROOFLINE_GRAPH // R} "
                            f"passes over {R} replicas)"},
        step_hbm_frac=per_launch / (dt / K) / HBM_PEAK)


# ------------------------------------------------------------------ prefill


def bench_prefill(work, iters, replicas):
    import numpy as np
    import torch

    import linear_attention_causal_amd as gdn

    s, d = work.shape, work.data
    geom = geometry(gdn, s)
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
    nbytes = prefill_bytes(geom, T, N, 2)
    util, traffic = recorded_prefill(work.name)
    return {"workload": work.name, "tokens": T, "sequences": N, "calls": iters,
            "ms_per_call": ms, "tokens_per_s": T / (ms * 1e-3),
            "roofline": {"bound": "hbm", "achieved": nbytes / (ms * 1e-3) / 1e9,
                         "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                         "frac": nbytes / (ms * 1e-3) / HBM_PEAK, "traffic": traffic,
                         "traffic_unit": "HBM bytes per call (scaled FETCH_SIZE + WRITE_SIZE "
                                         "over the call's kernels)",
                         "bytes_per_call": nbytes,
                         "timing": f"median over {iters} calls, HIP events on the launch stream"},
            "mfma": {"algorithmic_tflops": flops / (ms * 1e-3) / 1e12,
                     "algorithmic_frac_of_bf16_peak": flops / (ms * 1e-3) / BF16_PEAK,
                     "flop_per_call": flops,
                     "pipe_util_pct": util,
                     "pipe_util_source": "rocprofv3 MfmaUtil, kernel-time weighted over the "
                                         "call (committed prefill profile record; null once "
                                         "the kernels change)",
                     "dtype": "bf16 x3 on the state path (hi/lo split operands, f32 "
                              "accumulate), x1 on the output-only products"}}


# ------------------------------------------------------------------ block


def _graph_us(fn, R, warm=2, reps=20):
    """Median device time (us) of one of R back-to-back calls fn(r), captured
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
    geom = geometry(gdn, s)
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


def bench_serving(steps=64, layers=48, B=256, P=320, event_every=16):
    """B rows through `layers` layers per step, the layer launches of a step
    captured once as a HIP graph and replayed; after every `event_every`
    steps a seeded half of the rows retire, the survivors are compacted into
    the prefix across all layers (gdn_state_compact) and as many new rows are
    admitted behind them with zeroed state (recurrent and conv), the device
    slot index rewritten in place.  Pools and inputs are drawn on the device
    from a seeded generator (their values do not affect timing; this
    schedule's parity is tested at full head count with host-drawn pools)."""
    import numpy as np
    import torch

    import linear_attention_causal_amd as gdn
    import workloads as wl

    s = wl.FULL_HEADS
    geom = geometry(gdn, s)
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
    # device-resident slot index: the captured step reads it, an event rewrites it in place
    slot_d = _t(live, torch.int32)
    ws = gdn.decode_workspace(geom, B)

    def layer_pass(st):
        for L in Ls:
            gdn.gdn_decode_step(geom, L["w"], L["pool"], slot_d, x, z, a, b, y, ws, stream=st)

    events = []

    def event(live):
        keep, new_slots, src, dst = wl.retire_plan(rng, live, P)
        e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        e0.record(stream)
        if src.size:
            gdn.gdn_state_compact(geom, pools, src, dst, _t(src, torch.int32),
                                  _t(dst, torch.int32), stream=stream)
        e1.record(stream)
        n_keep = len(new_slots)
        n_new = len(live) - n_keep
        for L in Ls:                      # admitted rows start from zero state
            L["rec"][n_keep:n_keep + n_new].zero_()
            L["conv"][n_keep:n_keep + n_new].zero_()
        e2.record(stream)
        events.append((e0, e1, e2, int(src.size), n_new))
        live = np.concatenate([new_slots, np.arange(n_keep, n_keep + n_new)]).astype(np.int32)
        slot_d.copy_(torch.from_numpy(live))
        return live

    graph = capture(layer_pass)
    graph.replay()
    torch.cuda.synchronize()
    step_ev = []
    t0 = time.perf_counter()
    for t in range(steps):
        if t > 0 and t % event_every == 0:
            live = event(live)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        graph.replay()
        e1.record(stream)
        step_ev.append((e0, e1))
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    step_ms = [a_.elapsed_time(b_) for a_, b_ in step_ev]
    launch_us = float(np.median(step_ms)) * 1e3 / layers
    per_launch = step_bytes(geom, B, 2)
    per_step = layers * per_launch
    return {"workload": f"decode_b{B}_hk16_hv32_d128_p{P}_x{layers}layers",
            "launch": f"HIP graph of the {layers} layer launches per step, replayed",
            "steps": steps, "tokens_per_s": B * steps / dt, "ms_per_step": dt * 1e3 / steps,
            "hbm_frac_algorithmic": per_step * steps / dt / HBM_PEAK,
            "events": [{"after_step": event_every * (i + 1), "pairs_moved": n,
                        "admitted": adm, "compaction_ms": e0.elapsed_time(e1),
                        "admission_zeroing_ms": e1.elapsed_time(e2)}
                       for i, (e0, e1, e2, n, adm) in enumerate(events)],
            "roofline": {"bound": "hbm", "achieved": per_launch / (launch_us * 1e-6) / 1e9,
                         "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                         "frac": per_launch / (launch_us * 1e-6) / HBM_PEAK,
                         "traffic": recorded_traffic(SERVING_RECORD),
                         "traffic_unit": "HBM bytes per launch (scaled FETCH_SIZE + WRITE_SIZE)",
                         "kernel": "gdn::decode_head_kernel<__bf16, 128, 4>",
                         "bytes_per_launch": per_launch, "mean_launch_us": launch_us,
                         "timing": f"median over the {steps} replayed steps of HIP events on "
                                   f"the launch stream, / {layers} launches"}}


# ------------------------------------------------------------------ CPU oracle


def host_info():
    import platform
    model = platform.processor() or ""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count()
    return {"cpu_model": model, "host_cpus": os.cpu_count(), "cpus_available": avail}


def _rate(fn, units, budget):
    """units per second of fn() repeated for about `budget` seconds (at least once)."""
    n = 0
    t0 = time.perf_counter()
    while True:
        fn()
        n += 1
        dt = time.perf_counter() - t0
        if dt >= budget:
            return units * n / dt, n, dt


def cpu_baselines(budget, gpu=None):
    """The oracle as it stands (f64, C, one thread per independent (sequence
    or row, V-head) unit) on bounded samples of every workload, at one thread
    and at all the threads it uses.  Returns (headline entry, list)."""
    import numpy as np

    import oracle
    import workloads as wl

    info = host_info()
    nthr = oracle.default_threads()
    gpu = gpu or {}

    def og(s):
        return oracle.Geometry(s.num_k_heads, s.num_v_heads, s.head_k_dim, s.head_v_dim,
                               s.conv_kernel)

    def ow(w):
        return oracle.Weights(w["conv_w"], w["A_log"], w["dt_bias"], w["norm_w"])

    out = []

    def entry(name, unit, fns, sample, gpu_val=None):
        """fns: threads -> (callable, units per call)."""
        res = {"workload": name, "unit": unit, "sample": sample}
        for key, thr in (("all_threads", nthr), ("one_thread", 1)):
            fn, units = fns(thr)
            v, n, dt = _rate(fn, units, budget)
            res[key] = {"value": v, "threads": thr, "calls": n, "seconds": dt}
        if gpu_val is not None:
            res["gpu_value"] = gpu_val
            res["gpu_over_oracle_all_threads"] = gpu_val / res["all_threads"]["value"]
        out.append(res)
        log(f"[bench] oracle {name}: {res['all_threads']['value']:.4g} {unit} "
            f"({nthr} threads), {res['one_thread']['value']:.4g} (1 thread)")
        return res

    # tiny f32 layer: the whole workload (64-token prefill + 8 decode steps)
    wk = wl.tiny(seed=0)
    d = wk.data
    g1, w1 = og(wk.shape), ow(d["weights"])

    def tiny_fns(thr):
        def f():
            S, W = d["rec"].astype(np.float64), d["conv"].astype(np.float64)
            pre = d["prefill"]
            oracle.pool_run(g1, w1, S, W, d["cu_seqlens"], d["slot_idx"], pre["x"], pre["z"],
                            pre["a"], pre["b"], nthreads=thr)
            for st in d["steps"]:
                oracle.pool_run(g1, w1, S, W, [0, 1], d["slot_idx"], st["x"], st["z"], st["a"],
                                st["b"], nthreads=thr)
        return f, 64 + len(d["steps"])
    entry(wk.name, "tokens/s", tiny_fns, "the whole workload: 64-token prefill then 8 "
          "decode steps, Hk=2, Hv=4, d=32")

    # headline: decode steps of 16 rows
    wk = wl.decode_batch(seed=0)
    d = wk.data
    g2, w2 = og(wk.shape), ow(d["weights"])
    S2, W2 = d["rec"].astype(np.float64), d["conv"].astype(np.float64)
    B = len(d["slot_idx"])

    def dec_fns(thr):
        return (lambda: oracle.pool_run(g2, w2, S2, W2, np.arange(B + 1), d["slot_idx"], d["x"],
                                        d["z"], d["a"], d["b"], nthreads=thr)), B
    head = entry(wk.name, "tokens/s", dec_fns, "repeated decode steps of the 16 rows "
                 "(Hk=8, Hv=16, d=128), one step = 16 tokens", gpu.get("decode"))

    # 4096-token prefill: all heads; one thread on the first 512 tokens
    wk = wl.prefill_single(seed=0)
    d = wk.data
    g3, w3 = og(wk.shape), ow(d["weights"])

    def pre_fns(thr):
        T = 4096 if thr > 1 else 512
        S0, W0 = d["rec"].astype(np.float64), d["conv"].astype(np.float64)
        return (lambda: oracle.sequences(g3, w3, [0, T], d["x"][:T], d["z"][:T], d["a"][:T],
                                         d["b"][:T], S0, W0, nthreads=thr)), T
    entry(wk.name, "tokens/s", pre_fns, "all threads: the whole 4096-token call; one thread: "
          "its first 512 tokens (the token loop's cost per token is constant)",
          gpu.get(wk.name))

    # 8-sequence varlen prefill: the first tokens of every sequence
    wk = wl.prefill_varlen(seed=0)
    d = wk.data
    g5, w5 = og(wk.shape), ow(d["weights"])
    cu = d["cu_seqlens"]

    def var_fns(thr):
        n = 512 if thr > 1 else 32
        lens = [min(n, int(cu[i + 1] - cu[i])) for i in range(len(cu) - 1)]
        idx = np.concatenate([np.arange(cu[i], cu[i] + m) for i, m in enumerate(lens)])
        cu_s = np.concatenate([[0], np.cumsum(lens)])
        S0, W0 = d["rec"].astype(np.float64), d["conv"].astype(np.float64)
        return (lambda: oracle.sequences(g5, w5, cu_s, d["x"][idx], d["z"][idx], d["a"][idx],
                                         d["b"][idx], S0, W0, nthreads=thr)), idx.size
    entry(wk.name, "tokens/s", var_fns, "the first 512 tokens (or all, if fewer) of each of "
          "the 8 sequences with all threads, the first 32 with one; Hk=16, Hv=32, d=128, "
          "with their initial states", gpu.get(wk.name))

    # serving step: 256 rows x 48 layers + one compaction event; sampled on
    # whole layer-steps of one layer's pool and one layer's compaction, scaled
    s4 = wl.FULL_HEADS
    rng = np.random.default_rng(0)
    w4 = ow(wl.layer_weights(rng, s4))
    g4 = og(s4)
    P4, B4, L4 = 320, 256, 48
    S4 = (rng.standard_normal((P4, s4.num_v_heads, s4.head_k_dim, s4.head_v_dim)) * 0.1)
    W4 = rng.standard_normal((P4, s4.conv_kernel, s4.channels)) * 0.1
    live = rng.choice(P4, B4, replace=False).astype(np.int32)
    inp = wl.token_inputs(rng, s4, B4)
    _, _, src, dst = wl.retire_plan(rng, live, P4)

    def srv_fns(thr):
        rows = B4 if thr > 1 else 16
        def f():
            oracle.pool_run(g4, w4, S4, W4, np.arange(rows + 1), live[:rows], inp["x"][:rows],
                            inp["z"][:rows], inp["a"][:rows], inp["b"][:rows], nthreads=thr)
        return f, rows
    srv = entry(f"decode_b{B4}_hk16_hv32_d128_p{P4}_x{L4}layers", "tokens/s (one layer)",
                srv_fns, "layer-steps of one 320-slot pool (all 256 rows with all threads, 16 "
                "rows with one); a 48-layer step costs 48 of them, so its tokens/s is this "
                "value / 48, reported as `value_48_layers`", None)
    for key in ("all_threads", "one_thread"):
        srv[key]["value_48_layers"] = srv[key]["value"] / L4
    t0 = time.perf_counter()
    oracle.compact(g4, S4, W4, src, dst)
    srv["compaction_event_s"] = {"one_layer": time.perf_counter() - t0,
                                 "pairs": int(src.size), "layers_scaled": L4}
    srv["compaction_event_s"]["all_layers"] = srv["compaction_event_s"]["one_layer"] * L4
    if gpu.get("serving") is not None:
        srv["gpu_value"] = gpu["serving"]
        srv["gpu_over_oracle_all_threads"] = gpu["serving"] / srv["all_threads"]["value_48_layers"]
    del S4, W4

    hv = head["all_threads"]
    line = {"value": hv["value"], "unit": "tokens/s", "cores": hv["threads"], "kind": "oracle",
            "single_thread_value": head["one_thread"]["value"],
            "sample": f"{hv['calls']} decode steps of the headline workload (16 rows x 16 "
                      f"V-heads, d=128) in {hv['seconds']:.1f} s, f64, {hv['threads']} threads "
                      f"(one per (row, V-head) unit, at most 16); one thread: "
                      f"{head['one_thread']['calls']} steps",
            **info}
    return line, out


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch

    import linear_attention_causal_amd as gdn
    import workloads as wl

    gdn.library()
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    legs = set(args.legs.split(",")) if not args.no_extras else set()
    bad = legs - set(LEGS)
    if bad:
        print(f"unknown legs {sorted(bad)}", file=sys.stderr)
        sys.exit(2)
    if args.calibration_copy:
        calibration_copy()
    if args.calibration_gemm:
        calibration_gemm()
    if args.prefill_only:
        out = [bench_prefill(wl.prefill_single(seed=0), args.prefill_iters, replicas=6)]
        torch.cuda.empty_cache()
        out.append(bench_prefill(wl.prefill_varlen(seed=0), args.prefill_iters, replicas=1))
        print(json.dumps({"prefill": out}), flush=True)
        return
    if args.block_only:
        out = [bench_block(16, wl.RANK_LOCAL, 64, args.replicas)]
        torch.cuda.empty_cache()
        out.append(bench_block(256, wl.FULL_HEADS, 320, 4))
        print(json.dumps({"block": out}), flush=True)
        return
    log("[bench] decode headline")
    dec = bench_decode(args)
    torch.cuda.empty_cache()
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
        "timed_region": dec["timed_region"],
        "eager": dec["eager"],
        "step_hbm_frac_algorithmic": dec["step_hbm_frac"],
        "roofline": dec["roofline"],
    }
    gpu_vals = {"decode": dec["tokens_per_s"]}
    if "prefill" in legs:
        log("[bench] prefill t4096")
        pre = [bench_prefill(wl.prefill_single(seed=0), args.prefill_iters, replicas=6)]
        torch.cuda.empty_cache()
        log("[bench] prefill varlen8")
        pre.append(bench_prefill(wl.prefill_varlen(seed=0), args.prefill_iters, replicas=1))
        torch.cuda.empty_cache()
        line["prefill"] = pre
        for p in pre:
            gpu_vals[p["workload"]] = p["tokens_per_s"]
    if "block" in legs:
        log("[bench] decode block b16")
        line["block"] = [bench_block(16, wl.RANK_LOCAL, 64, args.replicas)]
        torch.cuda.empty_cache()
        log("[bench] decode block b256")
        line["block"].append(bench_block(256, wl.FULL_HEADS, 320, 4))
        torch.cuda.empty_cache()
    if "serving" in legs:
        log("[bench] serving 48 layers")
        line["serving"] = bench_serving(steps=args.serving_steps)
        gpu_vals["serving"] = line["serving"]["tokens_per_s"]
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline")
        line["cpu_baseline"], line["cpu_baselines"] = cpu_baselines(args.cpu_seconds, gpu_vals)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
