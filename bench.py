"""Benchmark of the fused MoE layer forward on one MI355X.

Default workload: the Mixtral-8x7B-shaped layer (H 4096, I 14336, 8 experts,
top-2, SwiGLU) in FP8 e4m3 W8A8 (per-output-channel weight scales, dynamic
per-token activation scales) at T = 128 tokens, the largest decode batch
the layer is quoted at; T = 32 and the Qwen3.5-35B-A3B-shaped layer at
T = 8192 (128x128 weight blocks, 1x128 activation groups) are timed in the
same run as further points of the metric.  A step is one moe_layer_forward
call: routing, dispatch, input quantisation, fused gate/up + SwiGLU grouped
GEMM, requantisation, down grouped GEMM and combine, on inputs already
resident in HBM.  The K timed calls are captured in one hipGraph and
replayed once, as a model step holds its layers in one graph; the same K
calls issued one launch per call (a graph each at decode sizes) are
reported beside it ("layer_us_one_launch_per_call"), and so are the calls
timed one at a time with HIP events, a 512 MiB buffer read between them so
the weights start from HBM rather than the 256 MB last-level cache
("layer_us_single_cold_llc": median, p10, p90).

Printed: one JSON line.  `value` is the algorithmic HBM throughput of the
layer (GB/s): bytes the method must move (weights and scales of the experts
that receive tokens, x read once, y written once, the FP8 intermediate
written and read once) over the measured time per step.  Also reported:
layer microseconds, active TFLOP/s (6*H*I*rows) and their fraction of the
FP8 MFMA peak, the roofline of the dominant kernel (its duration measured
with HIP events recorded around it on the launch stream, eager path, right
after the timed steps), and the CPU oracle timed on a bounded sample of the
same batch.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("MoE layer µs + active TFLOP/s / HBM GB/s (FP8 W8A8) at 32, 128, 8192 tokens")

# HBM bytes per launch of the dominant kernel measured with rocprofv3
# FETCH_SIZE / WRITE_SIZE counters, scaled by the same counters on a plain
# copy of known size (profiles/mixtral_fp8_T128_traffic_counters.md).  A
# figure is only reported while the kernel sources still hash to the value
# they had when the counters were taken.
TRAFFIC = {
    ("mixtral", 128, 2): {"bytes": 962571010, "src_sha": "094c15288b0b6928"},
}
KERNEL_SRC = ["grouped_gemm_amd/csrc/gemm_pipe.hip", "grouped_gemm_amd/csrc/common.h",
              "grouped_gemm_amd/csrc/layer.h"]


def kernel_src_sha() -> str:
    import hashlib
    data = b"".join(open(os.path.join(ROOT, f), "rb").read() for f in KERNEL_SRC)
    return hashlib.sha256(data).hexdigest()[:16]
HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5000.0
BF16_PEAK_TFLOPS = 2500.0
STAGES = ["route+dispatch", "quant_x", "gemm_gateup_swiglu", "quant_h", "gemm_down", "combine",
          "fused_decode_layer"]
# expert activations (include/moe.h MOE_ACT_*)
ACTIVATIONS = {"swiglu": 0, "swiglu_bounded": 1, "swiglu_oai": 2, "geglu": 3, "reglu": 4,
               "relu2": 5}
ACT_RELU2 = 5


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def layer_bytes(sh, T, n_active):
    """Algorithmic bytes of one layer call (see module docstring) and of one
    launch of the gate/up kernel; also the number of expert rows."""
    H, I = sh.hidden, sh.inter
    wbits = {0: 16, 1: 8, 2: 8, 3: 4}[sh.w_format]
    abytes = 2 if sh.a_format == 0 else 1

    def mat_scales(n, k):           # weight scale bytes of one [n, k] matrix
        return {0: 0, 1: n * 4, 2: (n // 128) * (k // 128) * 4, 3: n * k // 32}[sh.w_format]

    def act_scales(rows, k):        # activation scale bytes of [rows, k]
        return rows * {0: 0, 1: 4, 2: (k // 128) * 4, 3: k // 32}[sh.a_format]

    groups = n_active + sh.shared
    rows = T * sh.top_k + (T if sh.shared else 0)
    nmat = 1 if sh.activation == ACT_RELU2 else 2      # ReLU^2: no gate projection
    gateup = groups * nmat * (H * I * wbits / 8 + mat_scales(I, H))
    down = groups * (H * I * wbits / 8 + mat_scales(H, I))
    x_in = T * H * 2                                   # bf16 x read once
    y_out = T * H * 2                                  # bf16 y written once
    h_rt = 2 * (rows * I * abytes + act_scales(rows, I))
    total = gateup + down + x_in + y_out + h_rt
    g1 = gateup + T * H * abytes + act_scales(T, H) + rows * I * abytes + act_scales(rows, I)
    return total, g1, rows


FUSED_DECODE = False   # --fused-decode: the single-launch decode layer for T <= 16


def setup(name, T, seed_dev="cuda", act=0, bf16=False):
    import torch
    import grouped_gemm_amd as g
    import moe_synth as ms
    sh = ms.CONFIGS[name].with_(activation=act)
    if bf16:   # the same shape with bf16 weights and activations
        sh = sh.with_(w_format=ms.W_BF16, a_format=ms.A_BF16)
    B = ms.gen_batch(sh, T)
    # experts that receive tokens (stable argsort of the scores, top k)
    order = np.argsort(-B.scores.astype(np.float64), axis=1, kind="stable")[:, :sh.top_k]
    active = sorted(set(order.ravel().tolist()))
    t0 = time.time()
    W = ms.gen_weights(sh, experts=active)
    log(f"[bench] {name} T={T}: {len(active)} active experts, weights drawn in "
        f"{time.time() - t0:.1f}s")
    dW = {n: (torch.from_numpy(np.ascontiguousarray(getattr(W, n))).to(seed_dev)
              if getattr(W, n) is not None else None)
          for n in ("w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down",
                    "sh_gate", "sh_up", "sh_down", "ss_gate", "ss_up", "ss_down")}
    if act == ACT_RELU2:    # two-weight form: the gate weights are not passed
        for n in ("w_gate", "s_gate", "sh_gate", "ss_gate"):
            dW[n] = None
    ws = g.Workspace(sh.hidden, sh.inter, sh.experts, sh.top_k, T, shared_experts=sh.shared,
                     shared_inter=sh.shared_inter, score_fn=sh.score_fn, w_format=sh.w_format,
                     a_format=sh.a_format, activation=sh.activation, act_limit=sh.act_limit)
    if FUSED_DECODE:
        ws.set_fused_decode(True)
    x = torch.from_numpy(B.x_bits.view(np.int16)).to(seed_dev)
    s = torch.from_numpy(B.scores).to(seed_dev)
    y = torch.empty(T, sh.hidden, dtype=torch.int16, device=seed_dev)
    return sh, B, W, dW, ws, x, s, y, len(active)


def time_point(name, T, steps, warmup, force_cfg=-1, act=0, bf16=False):
    import torch
    import grouped_gemm_amd as g
    sh, B, W, dW, ws, x, s, y, n_active = setup(name, T, act=act, bf16=bf16)
    if force_cfg >= 0:
        ws.force_config(force_cfg)
    stream = torch.cuda.Stream()
    # warm-up: at least `warmup` calls and 0.2 s of them, so clocks and
    # caches settle before the first timed point
    with torch.cuda.stream(stream):
        n, t_w = 0, time.perf_counter()
        while n < warmup or time.perf_counter() - t_w < 0.2:
            g.layer_forward(ws, dW, x, s, y, stream=stream)
            n += 1
            if n % 16 == 0:
                stream.synchronize()
    torch.cuda.synchronize()
    # (a) one launch per layer call (a graph of its own at decode sizes)
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        for _ in range(steps):
            g.layer_forward(ws, dW, x, s, y, stream=stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_call = (t1 - t0) * 1e3 / steps
    # (b) the K layer calls captured in one graph and replayed once, as a
    # model step holds its layers in one graph: the host/command-processor
    # cost of launching a graph is paid once, not per layer
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for _ in range(steps):
            g.layer_forward(ws, dW, x, s, y, stream=stream)
    graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    graph.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / steps
    del graph
    cfg = ws.last_config(stream)
    # (c) the same calls timed one by one with events on the launch stream,
    # a 512 MiB scratch buffer read between them (outside the timed region;
    # read, not written, so no dirty lines are left to write back during
    # the call) so the weights do not sit in the 256 MB last-level cache:
    # median, p10 and p90
    flush = torch.ones(512 * 1024 * 1024 // 4, dtype=torch.float32, device="cuda")
    flush_sum = torch.empty((), dtype=torch.float32, device="cuda")
    single = []
    with torch.cuda.stream(stream):
        for i in range(steps):
            torch.sum(flush, dim=0, out=flush_sum)
            b = torch.cuda.Event(enable_timing=True)
            e = torch.cuda.Event(enable_timing=True)
            b.record(stream)
            g.layer_forward(ws, dW, x, s, y, stream=stream)
            e.record(stream)
            single.append((b, e))
    torch.cuda.synchronize()
    single_us = np.array([b.elapsed_time(e) * 1e3 for b, e in single])
    del flush, flush_sum
    # per-stage durations, eager path, events on the launch stream
    evs = []
    with torch.cuda.stream(stream):
        for _ in range(steps):
            pair = []
            for st in range(len(STAGES)):
                b = torch.cuda.Event(enable_timing=True)
                e = torch.cuda.Event(enable_timing=True)
                b.record(stream)
                e.record(stream)
                ws.set_stage_events(st, b, e)
                pair.append((b, e))
            g.layer_forward(ws, dW, x, s, y, stream=stream)
            evs.append(pair)
    torch.cuda.synchronize()
    for st in range(len(STAGES)):
        ws.set_stage_events(st, None, None)
    stage_ms = [float(np.mean([p[st][0].elapsed_time(p[st][1]) for p in evs]))
                for st in range(len(STAGES))]
    total_b, g1_b, rows = layer_bytes(sh, T, n_active)
    flops = (4.0 if sh.activation == ACT_RELU2 else 6.0) * sh.hidden * sh.inter * rows
    us = ms_step * 1e3
    return dict(sh=sh, B=B, W=W, T=T, us=us, ms=ms_step, us_call=ms_call * 1e3,
                us_flushed=[float(np.percentile(single_us, q)) for q in (50, 10, 90)],
                gbs=total_b / (us * 1e-6) / 1e9,
                tflops=flops / (us * 1e-6) / 1e12, bytes=total_b, g1_bytes=g1_b, flops=flops,
                stage_ms=stage_ms, cfg=cfg, n_active=n_active, rows=rows)


def cpu_baseline(pt, n_tokens):
    """The oracle on `n_tokens` tokens of the timed batch (all of them by
    default), wall-clock around the layer call only, scaled to the batch."""
    import oracle
    sh, B, W, T = pt["sh"], pt["B"], pt["W"], pt["T"]
    ids, w = oracle.route(B.scores, sh.top_k, sh.score_fn)
    n_tokens = T if n_tokens <= 0 else min(n_tokens, T)
    toks = np.linspace(0, T - 1, n_tokens).astype(np.int32)
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    threads = int(os.environ.get("OMP_NUM_THREADS", cores))
    t0 = time.perf_counter()
    oracle.layer_forward(W, B.x_bits, ids, w, tokens=toks)
    dt = time.perf_counter() - t0
    full = dt * T / n_tokens
    what = (f"all {T} tokens of the timed batch" if n_tokens == T else
            f"{n_tokens} of the {T} tokens of the timed batch, scaled to the full batch")
    return {"value": round(pt["bytes"] / full / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{what} (same weights, routing and activations), {dt:.1f}s wall "
                      f"({full:.2f}s per layer call)"}


def config_sweep(name, T, act=0, rounds=3, calls=30):
    """Median µs per layer call (eager, one launch sequence per call) for the
    device's own configuration choice and for every forced configuration,
    interleaved over `rounds` rounds after at least one second of warm-up
    (the best median of each is kept; the first calls after the weights are
    placed run several percent slower)."""
    import torch
    import grouped_gemm_amd as g
    sh, B, W, dW, ws, x, s, y, n_active = setup(name, T, act=act)
    ws.set_graphs(False)
    ncfg = 4
    st = torch.cuda.Stream()

    def median_us(n):
        with torch.cuda.stream(st):
            ts = []
            for _ in range(n):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(st)
                g.layer_forward(ws, dW, x, s, y, stream=st)
                e1.record(st)
                e1.synchronize()
                ts.append(e0.elapsed_time(e1) * 1e3)
        return float(np.median(ts))

    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 1.0:  # clocks and caches settle first
        median_us(10)
    best, chosen = {}, None
    for r in range(rounds):
        order = [-1] + list(range(ncfg))
        for c in (order if r % 2 == 0 else order[::-1]):
            ws.force_config(c)
            median_us(3)
            us = median_us(calls)
            best[c] = min(best.get(c, 1e30), us)
            if c < 0:
                chosen = ws.last_config()
    ws.force_config(-1)
    fastest = min(range(ncfg), key=lambda c: best[c])
    return {"workload": name, "tokens": T, "auto_config": chosen, "auto_us": round(best[-1], 1),
            "forced_us": {str(c): round(best[c], 1) for c in range(ncfg)},
            "fastest_config": fastest, "auto_over_fastest": round(best[-1] / best[fastest] - 1, 4)}


def config_sweep_many(name, tokens, act=0, rounds=3, calls=20, bf16=False):
    """config_sweep at several token counts of one workload with one weight
    draw (every expert), also reporting the routing histogram each point ran
    (the data the tile-configuration cost model is fitted to)."""
    import torch
    import grouped_gemm_amd as g
    import moe_synth as ms
    import oracle
    sh = ms.CONFIGS[name].with_(activation=act)
    if bf16:   # the same shape with bf16 weights and activations
        sh = sh.with_(w_format=ms.W_BF16, a_format=ms.A_BF16)
    t0 = time.time()
    W = ms.gen_weights(sh)
    log(f"[sweep] {name}: all {sh.experts} experts drawn in {time.time() - t0:.1f}s")
    dW = {n: (torch.from_numpy(np.ascontiguousarray(getattr(W, n))).cuda()
              if getattr(W, n) is not None else None)
          for n in ("w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down",
                    "sh_gate", "sh_up", "sh_down", "ss_gate", "ss_up", "ss_down")}
    del W
    ncfg = 4
    st = torch.cuda.Stream()
    out = []
    for T in tokens:
        B = ms.gen_batch(sh, T)
        ids, _ = oracle.route(B.scores, sh.top_k, sh.score_fn)
        counts = np.bincount(ids.ravel(), minlength=sh.experts).tolist()
        if sh.shared:
            counts.append(T)
        ws = g.Workspace(sh.hidden, sh.inter, sh.experts, sh.top_k, T, shared_experts=sh.shared,
                         shared_inter=sh.shared_inter, score_fn=sh.score_fn,
                         w_format=sh.w_format, a_format=sh.a_format, activation=sh.activation,
                         act_limit=sh.act_limit)
        ws.set_graphs(False)
        x = torch.from_numpy(B.x_bits.view(np.int16)).cuda()
        sc = torch.from_numpy(B.scores).cuda()
        y = torch.empty(T, sh.hidden, dtype=torch.int16, device="cuda")

        def median_us(n):
            with torch.cuda.stream(st):
                ts = []
                for _ in range(n):
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record(st)
                    g.layer_forward(ws, dW, x, sc, y, stream=st)
                    e1.record(st)
                    e1.synchronize()
                    ts.append(e0.elapsed_time(e1) * 1e3)
            return float(np.median(ts))

        tw = time.perf_counter()
        while time.perf_counter() - tw < 0.3:
            median_us(5)
        # -1: the library's choice with the cost model (default); -2: with
        # the fixed histogram rule; 0..: each configuration forced
        best, chosen = {}, {}
        for r in range(rounds):
            order = [-1, -2] + list(range(ncfg))
            for c in (order if r % 2 == 0 else order[::-1]):
                ws.set_config_model(c != -2)
                ws.force_config(max(c, -1))
                median_us(2)
                best[c] = min(best.get(c, 1e30), median_us(calls))
                if c < 0:
                    chosen[c] = ws.last_config()
        ws.set_config_model(True)
        ws.force_config(-1)
        fastest = min(range(ncfg), key=lambda c: best[c])
        rec = {"workload": name, "tokens": T, "hidden": sh.hidden, "inter": sh.inter,
               "experts": sh.experts, "top_k": sh.top_k, "shared": sh.shared,
               "w_format": sh.w_format, "counts": counts, "auto_config": chosen[-1],
               "auto_us": round(best[-1], 2), "candidates": ws.candidates(T),
               "rule_config": chosen[-2], "rule_us": round(best[-2], 2),
               "forced_us": {str(c): round(best[c], 2) for c in range(ncfg)},
               "fastest_config": fastest}
        log(f"[sweep] {name} T={T}: {rec['forced_us']} model {chosen[-1]} rule {chosen[-2]}")
        print(json.dumps(rec), flush=True)
        out.append(rec)
        del ws
    return out


BWD_STAGES = {7: "recompute_gate_up", 8: "input_grad_down", 9: "slot_pass",
              10: "input_grad_gate_up", 11: "input_grad_combine", 12: "weight_grad_down",
              13: "weight_grad_gate_up"}


def bench_backward(name="qwen", T=8192, steps=20, warmup=5):
    """Backward of the routed expert layer in bf16 (moe_expert_backward) on
    the named layer shape: whole-call time with HIP events, then each stage
    between events on the launch stream.  Useful FLOPs: 12 H I per slot (the
    input and weight gradients of three projections; the gate/up
    recomputation, another 4 H I per slot, is not counted)."""
    import torch
    import grouped_gemm_amd as g
    import moe_synth as ms
    import oracle
    sh = ms.CONFIGS[name].with_(w_format=ms.W_BF16, a_format=ms.A_BF16)
    B = ms.gen_batch(sh, T)
    ids, w = oracle.route(B.scores, sh.top_k, sh.score_fn)
    act_e = sorted(set(np.unique(ids).tolist()))
    t0 = time.time()
    W = ms.gen_weights(sh, experts=act_e)
    log(f"[bench] backward {name} T={T}: {len(act_e)} active experts, weights drawn in "
        f"{time.time() - t0:.1f}s")
    dW = {n: torch.from_numpy(np.ascontiguousarray(getattr(W, n)).view(np.int16)).cuda()
          for n in ("w_gate", "w_up", "w_down")}
    del W
    ws = g.Workspace(sh.hidden, sh.inter, sh.experts, sh.top_k, T, score_fn=sh.score_fn,
                     w_format=sh.w_format, a_format=sh.a_format)
    E, I, H, k = sh.experts, sh.inter, sh.hidden, sh.top_k
    x = torch.from_numpy(B.x_bits.view(np.int16)).cuda()
    dy = torch.from_numpy(ms.gen_grad(sh, T).view(np.int16)).cuda()
    tid = torch.from_numpy(ids.astype(np.int32)).cuda()
    tw = torch.from_numpy(w.astype(np.float32)).cuda()
    dx = torch.empty(T, H, dtype=torch.int16, device="cuda")
    dwg = torch.empty(E, I, H, device="cuda")
    dwu = torch.empty(E, I, H, device="cuda")
    dwd = torch.empty(E, H, I, device="cuda")
    dtw = torch.empty(T, k, device="cuda")
    scratch = torch.empty(g.backward_scratch_size(ws), dtype=torch.uint8, device="cuda")
    st = torch.cuda.Stream()

    def call():
        g.expert_backward(ws, dW, x, tid, tw, dy, dx, dwg, dwu, dwd, dtw, scratch, stream=st)

    with torch.cuda.stream(st):
        for _ in range(warmup):
            call()
        st.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(steps):
            call()
        e1.record(st)
        e1.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / steps
        evs = {sid: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for sid in BWD_STAGES}
        for a, b in evs.values():   # the events must exist before the library records them
            a.record(st)
            b.record(st)
        for sid, (a, b) in evs.items():
            ws.set_stage_events(sid, a, b)
        stage = {sid: 0.0 for sid in BWD_STAGES}
        for _ in range(steps):
            call()
            st.synchronize()
            for sid, (a, b) in evs.items():
                stage[sid] += a.elapsed_time(b) / steps
        for sid in BWD_STAGES:
            ws.set_stage_events(sid, None, None)
    S = T * k
    flops = 12.0 * H * I * S
    # FLOPs of the stages that are one kernel launch each
    per = {8: 2.0 * H * I * S, 10: 4.0 * H * I * S}
    dom = max(per, key=lambda sid: stage[sid])
    ach = per[dom] / (stage[dom] * 1e-3) / 1e12
    out = {"workload": f"{name}-shaped MoE expert layer backward, bf16, H{H} I{I} E{E} top{k}, T={T}",
           "us": round(us, 2), "tflops": round(flops / (us * 1e-6) / 1e12, 2),
           "bf16_mfma_frac": round(flops / (us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4),
           "stage_ms": {BWD_STAGES[sid]: round(v, 5) for sid, v in stage.items()},
           "roofline": {"bound": "mfma", "achieved": round(ach, 1), "peak": BF16_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(ach / BF16_PEAK_TFLOPS, 4),
                        "traffic": None, "kernel": BWD_STAGES[dom],
                        "avg_ms": round(stage[dom], 5), "flops_per_launch": per[dom]}}
    log(f"[bench] backward {name} T={T}: {us:.1f} us, {out['tflops']:.1f} TFLOP/s "
        f"({out['bf16_mfma_frac']:.3f} of bf16 peak), stages(ms)="
        f"{[round(v, 4) for v in stage.values()]}")
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mixtral")
    ap.add_argument("--tokens", type=int, default=0)
    ap.add_argument("--cpu-tokens", type=int, default=0,
                    help="tokens of the batch the CPU oracle is timed on (0: all)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the 8192-token Qwen-shaped point of the default run")
    ap.add_argument("--no-decode-extra", action="store_true",
                    help="skip the DeepSeek-V3-shaped T=1/16 points of the default run")
    ap.add_argument("--force-config", type=int, default=-1,
                    help="tile configuration (default: chosen on the device)")
    ap.add_argument("--activation", default="swiglu", choices=list(ACTIVATIONS),
                    help="expert activation of every timed point (default SwiGLU)")
    ap.add_argument("--bf16", action="store_true",
                    help="run the workload's shape with bf16 weights and activations")
    ap.add_argument("--config-sweep", action="store_true",
                    help="time the device's configuration choice against every forced "
                         "configuration at each token count of the workload (or --tokens) "
                         "and print one JSON line per point instead of the benchmark line")
    ap.add_argument("--sweep-tokens", default="",
                    help="with --config-sweep: comma-separated token counts timed with one "
                         "weight draw of every expert, printing the routing histogram of each")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain elementwise copy of 256 MiB (fp32 in, fp32 out), "
                         "whose known byte counts calibrate hardware traffic counters")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the backward point (Qwen-shaped bf16 expert layer, T=8192)")
    ap.add_argument("--backward-only", action="store_true",
                    help="time only the backward point and print its JSON object")
    ap.add_argument("--fused-decode", action="store_true",
                    help="run batches of at most 16 tokens through the single-launch decode layer")
    args = ap.parse_args()
    global FUSED_DECODE
    FUSED_DECODE = args.fused_decode
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the layer holds every expert on one device); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import grouped_gemm_amd  # noqa: F401  (fails loudly if the library is not built)

    import moe_synth as ms
    if args.copy_calibration:
        n = 64 * 1024 * 1024
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            torch.mul(a, 1.0, out=b)
        torch.cuda.synchronize()
        log(f"[bench] copy calibration: 3 x elementwise copy, {4 * n} bytes read and "
            f"{4 * n} bytes written per launch")
        del a, b
    act = ACTIVATIONS[args.activation]
    sh0 = ms.CONFIGS[args.workload]
    if args.config_sweep:
        if args.sweep_tokens:
            config_sweep_many(args.workload, [int(t) for t in args.sweep_tokens.split(",")], act,
                              bf16=args.bf16)
            return
        for T in ([args.tokens] if args.tokens else list(sh0.tokens)):
            print(json.dumps(config_sweep(args.workload, T, act)), flush=True)
        return
    if args.backward_only:
        print(json.dumps(bench_backward("qwen", args.tokens or 8192, args.steps, args.warmup)),
              flush=True)
        return
    T_main = args.tokens or max(sh0.tokens)
    points = []
    extra_T = [t for t in sh0.tokens if t != T_main] if not args.tokens else []
    for T in extra_T:
        p = time_point(args.workload, T, args.steps, args.warmup, args.force_config, act,
                       args.bf16)
        points.append(p)
        log(f"[bench] T={T}: {p['us']:.1f} us, {p['gbs']:.0f} GB/s, {p['tflops']:.2f} TFLOP/s")
    main_pt = time_point(args.workload, T_main, args.steps, args.warmup, args.force_config, act,
                         args.bf16)
    points.append(main_pt)
    log(f"[bench] T={T_main}: {main_pt['us']:.1f} us, {main_pt['gbs']:.0f} GB/s, "
        f"{main_pt['tflops']:.2f} TFLOP/s, stages(ms)={[round(v, 4) for v in main_pt['stage_ms']]}")
    if args.workload == "mixtral" and not args.tokens and not args.no_prefill:
        # the metric's 8192-token point: the Qwen3.5-35B-A3B-shaped layer
        qp = time_point("qwen", 8192, args.steps, args.warmup, act=act, bf16=args.bf16)
        points.append(qp)
        log(f"[bench] qwen T=8192: {qp['us']:.1f} us, {qp['gbs']:.0f} GB/s, "
            f"{qp['tflops']:.2f} TFLOP/s ({qp['tflops'] / FP8_PEAK_TFLOPS:.3f} of FP8 peak), "
            f"stages(ms)={[round(v, 4) for v in qp['stage_ms']]}")
    if args.workload == "mixtral" and not args.tokens and not args.no_decode_extra:
        # the DeepSeek-V3-shaped decode points (one and sixteen tokens)
        for T in (1, 16):
            dp = time_point("dsv3", T, args.steps, args.warmup, act=act, bf16=args.bf16)
            points.append(dp)
            log(f"[bench] dsv3 T={T}: {dp['us']:.1f} us, {dp['gbs']:.0f} GB/s "
                f"({dp['gbs'] / HBM_PEAK_GBS:.3f} of HBM), stages(ms)="
                f"{[round(v, 4) for v in dp['stage_ms']]}")
            del dp["W"], dp["B"]
    bwd = None
    if args.workload == "mixtral" and not args.tokens and not args.no_backward:
        bwd = bench_backward("qwen", 8192, args.steps, args.warmup)
    dom = int(np.argmax(main_pt["stage_ms"]))
    dom_ms = main_pt["stage_ms"][dom]
    if dom == 2:
        dom_bytes = main_pt["g1_bytes"]
    else:
        dom_bytes = None
    roof = None
    if dom_bytes is not None:
        ach = dom_bytes / (dom_ms * 1e-3) / 1e9
        tr = TRAFFIC.get((args.workload, T_main, main_pt["cfg"])) if act == 0 else None
        traffic = tr["bytes"] if tr and tr["src_sha"] == kernel_src_sha() else None
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": ("k_gemm_stream (gate/up + %s)" % args.activation if main_pt["cfg"] == 0
                           else "k_gemm_pipe (gate/up + %s, %d-row blocks)"
                           % (args.activation, {1: 32, 2: 64, 3: 128}.get(main_pt["cfg"], 0))),
                "avg_ms": round(dom_ms, 5),
                "bytes_per_launch": int(dom_bytes)}
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(main_pt, args.cpu_tokens)
        log(f"[bench] cpu oracle: {cpu}")
    sh = main_pt["sh"]
    out = {
        "metric": METRIC, "value": round(main_pt["gbs"], 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(main_pt["ms"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if args.bf16 else "fp8",
        "data": "synthetic",
        "config": {"workload": f"{sh.name}-shaped MoE layer H{sh.hidden} I{sh.inter} "
                               f"E{sh.experts} top{sh.top_k}, T={T_main}",
                   "tokens": T_main, "hidden": sh.hidden, "inter": sh.inter,
                   "experts": sh.experts, "top_k": sh.top_k, "w_format": sh.w_format,
                   "a_format": sh.a_format, "activation": args.activation,
                   "tile_config": main_pt["cfg"]},
        "points": [{"workload": p["sh"].name, "tokens": p["T"], "layer_us": round(p["us"], 2),
                    "layer_us_one_launch_per_call": round(p["us_call"], 2),
                    "layer_us_single_cold_llc": {"median": round(p["us_flushed"][0], 2),
                                                 "p10": round(p["us_flushed"][1], 2),
                                                 "p90": round(p["us_flushed"][2], 2)},
                    "active_tflops": round(p["tflops"], 3), "hbm_gbs": round(p["gbs"], 1),
                    "hbm_frac": round(p["gbs"] / HBM_PEAK_GBS, 4),
                    "fp8_mfma_frac": round(p["tflops"] / FP8_PEAK_TFLOPS, 4),
                    "bf16_mfma_frac": round(p["tflops"] / BF16_PEAK_TFLOPS, 4),
                    "stage_ms": {STAGES[i]: round(v, 5) for i, v in enumerate(p["stage_ms"])}}
                   for p in points],
        "roofline": roof,
        "cpu_baseline": cpu,
        "backward": bwd,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
