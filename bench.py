"""Benchmark of one NVFP4 sparse-MoE FFN layer on one MI355X.

A step is one pass of the whole layer over one batch of seeded synthetic tokens whose inputs
are already resident in HBM.  Prints one JSON line (the benchmark contract) with the layer
throughput; the roofline of the dominant kernel work, timed with HIP events on the launch
stream over the timed region; its HBM traffic from the committed PMC summary when the kernels
are unchanged since; and the CPU oracle timed on a bounded sample.  By default every workload below runs in turn, in one process: decode1 gives
the line's top-level fields and the others the same fields under "legs" (decode1, decode64 and
prefill16k share one generated expert set).  --workload runs one workload alone.

Up to 128 tokens a step is one moe_layer_nvfp4 call, timed with HIP events around the timed
steps: for one or two tokens a single persistent kernel, from three tokens the fused routing
kernel (router, top-k, grouping, tile plan in one launch), the expert FFN and the combine; the
roofline is then that of the whole layer.  Above 128 tokens the step is the four public calls,
with HIP events around the expert-FFN call (its roofline) and the combine call.

Warmup: the W warmup steps, then untimed steps until --settle-s seconds (default 0.3) of warmup
have passed: a GPU that was idle runs its first milliseconds of work at lower clocks, and a few
steps of a short workload do not cover that ramp.  The JSON line reports both counts.

--combine norm replaces the plain combine with the combine variants (per-expert RMS norm before
the weighted sum, then the residual update and the next layer's RMS norm) and runs the four-call
path at every T.

Workloads (hidden 7168, 256 experts, top-8, NVFP4 experts):
  decode1     T=1, expert intermediate 2048; each step takes the next token of a seeded pool of
              64 tokens, so consecutive steps read different experts (as decoding does) rather
              than re-reading a set that fits the 256 MB Infinity Cache   [headline]
  decode64    T=64, uniform-random router weights
  verify128   T=128 (8 requests x 16 draft positions), intermediate 256 (one 1/8 shard),
              Zipf(1.1) expert-popularity bias on the logits
  prefill16k  T=16384 (8 x 2048)
"""
import argparse
import json
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer tokens/s + achieved HBM GB/s (T=1,64) / MFMA util (T=16K)"
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
MFMA_F16_PEAK_TFS = 2500.0  # MI355X dense f16/bf16 matrix throughput
MFMA_F8_PEAK_TFS = 5000.0   # MI355X dense fp8 matrix throughput
POOL = 64


def expert_bytes(H, I):
    """packed e2m1 codes + e4m3 scales of gate, up and down of one expert"""
    return 3 * (H * I // 2 + H * I // 16)


def mx8_expert_bytes(H, I):
    """e4m3 codes + e8m0 scales (one per 32) of gate, up and down of one expert"""
    return 3 * (H * I + H * I // 32)


LEGS = ("decode1", "decode64", "verify128", "prefill16k")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="all", choices=("all",) + LEGS,
                    help="all (default): decode1 is the headline line, the other workloads are "
                         "reported under 'legs'; else that workload alone")
    ap.add_argument("--combine", default="plain", choices=["plain", "norm"],
                    help="plain: routing-weighted sum; norm: per-expert RMS norm before the sum "
                         "and the residual + next pre-norm epilogue (four-call path)")
    ap.add_argument("--precision", default="nvfp4", choices=["nvfp4", "mx8"],
                    help="mx8: the fp8-compute variant (MXFP8 weights requantised from NVFP4 at "
                         "load time, MXFP8 x and h, scaled matrix cores; four-call path)")
    ap.add_argument("--settle-s", type=float, default=0.3,
                    help="after the W warmup steps, keep running untimed steps until this many "
                         "seconds of warmup have passed, so the timed steps run at the clocks of "
                         "a busy GPU, not those of one that was idle (0 disables)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU oracle sample budget per workload (0 disables the CPU baseline)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(sharding is described in DESIGN.md). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    legs = LEGS if args.workload == "all" else (args.workload,)
    shared = {}
    results = {}
    for wl in legs:
        results[wl] = run_leg(wl, args, dev, shared)
        if wl != legs[0]:
            print("leg %s: %.2f us/layer, roofline frac %s" % (
                wl, results[wl]["us_per_layer"], results[wl]["roofline"]["frac"]),
                file=sys.stderr, flush=True)
    head = results[legs[0]]
    if len(legs) > 1:
        head["legs"] = {wl: leg_summary(results[wl]) for wl in legs[1:]}
    print(json.dumps(head))


def leg_summary(r):
    """The per-workload record under 'legs' of the headline line."""
    keep = ("value", "unit", "steps", "warmup", "settle_steps", "ms_per_step", "us_per_layer", "kernel_us",
            "dtype", "config", "roofline", "cpu_baseline", "distinct_experts", "layer_hbm_frac",
            "kernel_algorithmic_bytes", "combine", "ffn_flops")
    return {k: r[k] for k in keep if k in r}


def _experts(sp, dev, shared, seed=0):
    """Expert weights of a workload (row-major for the oracle's host copy, tile-major for the
    library), generated once per (H, I, E) and shared by the workloads of the same shape: the
    generator of every expert is seeded by (seed, expert) alone."""
    import bit_expert_ffn_amd as moe
    import synth
    key = (sp["E"], sp["H"], sp["I"], seed)
    if key not in shared:
        shared.clear()  # one weight set resident at a time
        torch.cuda.empty_cache()
        raw = synth.make_experts(sp["E"], sp["H"], sp["I"], seed, dev)
        shared[key] = {"raw": raw, "packed": moe.pack_experts(raw)}
    return shared[key]


def run_leg(wl, args, dev, shared):
    import bit_expert_ffn_amd as moe
    import synth

    sp = dict(synth.SPECS[wl])
    T, H, I, E, k = sp["T"], sp["H"], sp["I"], sp["E"], sp["k"]
    big = wl == "prefill16k"
    steps = args.steps if args.steps is not None else (10 if big else 200)
    warmup = args.warmup if args.warmup is not None else (3 if big else 20)

    print("generating %s inputs on the GPU" % wl, file=sys.stderr, flush=True)
    pool = POOL if T == 1 else 1
    seed = 0
    xs = synth.make_x(T * pool, H, seed, dev)
    wr = synth.make_router(H, E, sp.get("router", "normal"), seed, dev)
    bias = synth.make_zipf_bias(E, sp["zipf"], seed, dev) if sp.get("zipf") else None
    wset = _experts(sp, dev, shared, seed)
    layer = dict(spec=sp, x=xs, w_router=wr, bias=bias, experts=wset["raw"])
    mx8 = args.precision == "mx8"
    if mx8:  # load-time requantisation to MXFP8 (outside the timed region)
        ex = moe.mx8_experts(layer["experts"])
    else:
        ex = wset["packed"]  # tile-major copy (load-time conversion)
    buf = moe.LayerBuffers(T, H, I, E, k, device=dev, y_dtype=torch.float16, logits=False)
    torch.cuda.synchronize()

    def x_of(i):
        j = (i % pool) * T
        return xs[j:j + T]

    stream = torch.cuda.current_stream(dev)

    # up to 128 tokens the step is one moe_layer_nvfp4 call (plain combine only): for one or two
    # tokens a single persistent kernel, from three tokens the fused routing kernel (router,
    # top-k, grouping, tile plan), the expert FFN and the combine
    fused = T <= 128 and args.combine == "plain" and not mx8
    norm = args.combine == "norm"
    if norm:
        g = torch.Generator(device=dev)
        g.manual_seed(11)
        resid = torch.randn((T, H), generator=g, device=dev, dtype=torch.float32)
        gain = torch.rand((H,), generator=g, device=dev, dtype=torch.float32) + 0.5
        x_next = torch.empty((T, H), device=dev, dtype=torch.bfloat16)
    calls = ([moe.prepare_layer_nvfp4(x_of(i), wr, bias, ex, k, buf, stream=stream)
              for i in range(pool)] if fused else None)

    def step(i, ev=None, evc=None):
        x = x_of(i)
        if fused:
            if ev is not None:
                ev[0].record(stream)
            calls[i % pool]()
            if ev is not None:
                ev[1].record(stream)
            return
        moe.route(x, wr, bias, k, buf.topk_id, buf.topk_w, buf.ws, stream=stream)
        moe.group(buf.topk_id, E, buf.count, buf.offset, buf.sorted_slot, buf.slot_row,
                  buf.active, buf.n_active, buf.ws, stream=stream)
        if ev is not None:
            ev[0].record(stream)
        if mx8:
            moe.expert_ffn_mx8(x, ex, buf.count, buf.offset, buf.sorted_slot, buf.active,
                               buf.n_active, k, buf.y, buf.ws, stream=stream)
        else:
            moe.expert_ffn_nvfp4(x, ex, buf.count, buf.offset, buf.sorted_slot, buf.active,
                                 buf.n_active, k, buf.y, buf.ws, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        if evc is not None:
            evc[0].record(stream)
        if norm:  # the residual stream is updated in place
            moe.combine_norm(buf.y, buf.slot_row, buf.topk_w, resid, expert_norm=True,
                             resid=resid, alpha=1.0, beta=1.0, gain=gain, x_next=x_next,
                             stream=stream)
        else:
            moe.combine(buf.y, buf.slot_row, buf.topk_w, buf.out, stream=stream)
        if evc is not None:
            evc[1].record(stream)

    t_w = time.perf_counter()
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    # settle: a GPU that was idle (host-side setup, another workload's CPU baseline) runs its
    # first milliseconds of work at lower clocks; a few warmup steps of a short workload do not
    # cover that ramp, so untimed steps continue until settle_s seconds of warmup have passed
    settle = 0
    while time.perf_counter() - t_w < args.settle_s:
        for _ in range(8):
            step(warmup + settle)
            settle += 1
        torch.cuda.synchronize()
    print("%s: warmup done (%d steps + %d settle steps); timing %d steps" % (
        wl, warmup, settle, steps), file=sys.stderr, flush=True)

    # timed region: exactly `steps` layer calls, bracketed by device synchronisation
    # HIP events on the launch stream: around the expert-FFN call of every step (four-call
    # path), or around the whole run when a step is the single-launch kernel
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    evcs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(steps)]
    ev_all = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    n_distinct = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev_all[0].record(stream)
    for i in range(steps):
        step(warmup + i, None if fused else evs[i], None if fused else evcs[i])
    ev_all[1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    if fused:
        moe.layer_check(buf.ws, stream=stream)  # no wait of the single launch gave up
        ffn_ms = ev_all[0].elapsed_time(ev_all[1]) / steps
    else:
        ffn_ms = sum(a.elapsed_time(b) for a, b in evs) / steps
        comb_ms = sum(a.elapsed_time(b) for a, b in evcs) / steps

    # distinct experts touched per step (re-run routing+grouping outside the timed region)
    for i in range(min(steps, POOL if T == 1 else 1)):
        x = x_of(warmup + i)
        moe.route(x, wr, bias, k, buf.topk_id, buf.topk_w, buf.ws, stream=stream)
        moe.group(buf.topk_id, E, buf.count, buf.offset, buf.sorted_slot, buf.slot_row,
                  buf.active, buf.n_active, buf.ws, stream=stream)
        n_distinct.append(int(buf.n_active.item()))
    nd = sum(n_distinct) / len(n_distinct)

    ms_step = elapsed * 1e3 / steps
    tok_s = T * steps / elapsed
    w_bytes = nd * (mx8_expert_bytes(H, I) if mx8 else expert_bytes(H, I))
    ffn_bytes = w_bytes + T * H * 2 + T * k * H * 2          # weights + x + y (f16)
    layer_bytes = w_bytes + T * H * 2 + H * E * 4 + T * H * 4  # weights + x + router + out
    flops = 6.0 * T * k * H * I
    traffic = None
    if fused and T <= 2:
        # the single kernel reads the expert weights, x and the router weights, writes out
        kernel, kbytes = "layer_small_kernel", layer_bytes
        if wl == "decode1":
            traffic = measured_traffic("traffic_layer_small_decode1.txt")
    elif fused:
        # the whole layer: expert weights, x and router weights read, out written (y and the
        # routing arrays are intermediates)
        kernel, kbytes = ("moe_layer_nvfp4 (route_group_kernel, expert FFN, combine)",
                          layer_bytes)
        traffic = measured_traffic("traffic_layer_%s.txt" % wl)
    elif mx8:
        kernel, kbytes = "fp8 expert FFN call (x quantiser + two scaled-MFMA grouped GEMMs)", ffn_bytes
        traffic = measured_traffic("traffic_ffn_mx8_%s.txt" % wl)
    else:
        kernel, kbytes = "expert FFN call (few-row kernels + grouped GEMM)", ffn_bytes
        traffic = measured_traffic("traffic_ffn_%s.txt" % wl)
    if big:
        peak = MFMA_F8_PEAK_TFS if mx8 else MFMA_F16_PEAK_TFS
        achieved = flops / (ffn_ms * 1e-3) / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 2), peak=peak,
                    unit="TFLOP/s", frac=round(achieved / peak, 4), traffic=traffic,
                    kernel=kernel)
    else:
        achieved = kbytes / (ffn_ms * 1e-3) / 1e9
        roof = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4), traffic=traffic, kernel=kernel)

    combine = None
    if not fused:
        # y (f16) + slot_row + weights per token; plain: out fp32; norm: resid fp32 read,
        # new residual fp32 written, x_next bf16 written (gain [H] fp32 read once)
        cb = T * (k * H * 2 + k * 8) + (T * H * 10 + H * 4 if norm else T * H * 4)
        combine = dict(kernel="combine_norm_kernel" if norm else "combine_kernel",
                       variant="expert_norm+residual_norm" if norm else "plain",
                       us=round(comb_ms * 1e3, 2), algorithmic_bytes=int(cb),
                       achieved_gbs=round(cb / (comb_ms * 1e-3) / 1e9, 1),
                       frac=round(cb / (comb_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                       traffic=measured_traffic("traffic_%s_%s.txt" % (
                           "combine_norm" if norm else "combine", wl)))

    cpu = None
    if args.cpu_seconds > 0:
        cpu = (cpu_baseline_mx8(layer, sp, args.cpu_seconds) if mx8 else
               cpu_baseline(layer, sp, pool, args.cpu_seconds, shared))
        if norm:
            cpu["combine_norm"] = cpu_combine_norm(T, k, H, min(T, 256))
    del buf, calls
    torch.cuda.empty_cache()

    return {
        "metric": METRIC, "value": round(tok_s, 2), "unit": "tokens/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "settle_steps": settle, "settle_s": args.settle_s,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8 (e4m3, MX)" if mx8 else "f16",
        "data": "synthetic",
        "config": {"workload": wl, "T": T, "H": H, "I": I, "E": E, "k": k,
                   "combine": "expert_norm+residual_norm" if norm else "plain",
                   "weights": ("mxfp8 (e4m3, e8m0 per 32), requantised from nvfp4 at load"
                               if mx8 else "nvfp4 (e2m1, e4m3 per 16, fp32 per matrix)"),
                   "precision": args.precision,
                   "token_pool": pool, "seed": 0, "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "us_per_layer": round(ms_step * 1e3, 2),
        "kernel_us": round(ffn_ms * 1e3, 2),
        "distinct_experts": round(nd, 2),
        "layer_hbm_frac": round(layer_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "kernel_algorithmic_bytes": int(kbytes),
        "combine": combine,
        "ffn_flops": flops,
    }


def measured_traffic(kernel_file):
    """HBM bytes per launch from the committed PMC summary of this kernel, if the kernel's
    sources are unchanged since the counters were taken (else None)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", kernel_file)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line:
            key, val = line.split(":", 1)
            fields[key.strip()] = val.strip()
    try:
        h = hashlib.sha256()
        for src in fields["sources"].split():
            h.update(open(os.path.join(ROOT, src), "rb").read())
        if h.hexdigest() != fields["sha256"]:
            return None
        return int(fields["bytes_per_launch"])
    except (KeyError, OSError, ValueError):
        return None


def cpu_baseline(layer, sp, pool, budget_s, shared=None):
    """The oracle as it stands, on a bounded sample of the same workload: whole-layer output of
    as many tokens as fit the time budget (at least one), tokens/s."""
    import numpy as np
    import oracle
    print("copying inputs to the host for the CPU oracle", file=sys.stderr, flush=True)
    key = "host_experts"
    if shared is not None and key in shared and shared[key][0] is layer["experts"]:
        ex = shared[key][1]
    else:
        ex = oracle.Experts(**{n: v.cpu().numpy() for n, v in layer["experts"].items()})
        if shared is not None:
            shared[key] = (layer["experts"], ex)
    x = layer["x"].cpu().view(torch.int16).numpy().view(np.uint16)
    wr = layer["w_router"].cpu().numpy()
    bias = None if layer["bias"] is None else layer["bias"].cpu().numpy()
    done = 0
    t0 = time.perf_counter()
    while True:
        oracle.layer_tokens(x, wr, bias, ex, sp["k"], [done % x.shape[0]])
        done += 1
        if time.perf_counter() - t0 >= budget_s or done >= x.shape[0]:
            break
    dt = time.perf_counter() - t0
    return {"value": round(done / dt, 4), "unit": "tokens/s", "cores": oracle.threads(),
            "kind": "oracle",
            "sample": "%d token(s) of the %s workload (T=%d), whole layer per token (fp64 oracle)"
                      % (done, "decode" if pool > 1 else "same", sp["T"])}


def cpu_baseline_mx8(layer, sp, budget_s):
    """The oracle's fp8 variant on a bounded sample: per token, the oracle router and top-k, the
    MXFP8 requantisation of that token's k experts, their fp8 FFN rows and the weighted sum;
    tokens/s (the requantisation is counted: the oracle has no other way to get the weights)."""
    import numpy as np
    import oracle
    print("copying inputs to the host for the CPU oracle (fp8 variant)", file=sys.stderr,
          flush=True)
    x = layer["x"].cpu().view(torch.int16).numpy().view(np.uint16)
    wr = layer["w_router"].cpu().numpy()
    bias = None if layer["bias"] is None else layer["bias"].cpu().numpy()
    k = sp["k"]
    done = 0
    t0 = time.perf_counter()
    while True:
        t = done % x.shape[0]
        ids, w = oracle.topk(oracle.router(x[t:t + 1], wr, bias), k)
        sub = oracle.Experts(**{n: v[ids[0].tolist()].cpu().numpy()
                                for n, v in layer["experts"].items()})
        mx = oracle.nvfp4_to_mxfp8(sub)
        out = np.zeros(sp["H"])
        for j in range(k):
            out += w[0, j] * oracle.expert_rows_mx(x[t:t + 1], mx, j, [0])[0]
        done += 1
        if time.perf_counter() - t0 >= budget_s or done >= x.shape[0]:
            break
    dt = time.perf_counter() - t0
    return {"value": round(done / dt, 4), "unit": "tokens/s", "cores": oracle.threads(),
            "kind": "oracle",
            "sample": "%d token(s) of the workload, fp8 variant per token (router, top-k, MXFP8 "
                      "requantisation of its experts, fp8 FFN rows, weighted sum; fp64 oracle)"
                      % done}


def cpu_combine_norm(T, k, H, ntok):
    """The oracle's combine variants (per-expert norm + epilogue) on ntok tokens of seeded
    inputs of the workload's shape, tokens/s."""
    import oracle
    import synth
    d = {n: v.numpy() for n, v in synth.make_combine_inputs(ntok, k, H, seed=12).items()}
    t0 = time.perf_counter()
    oracle.combine_norm(d["y"].astype("float32"), d["slot_row"], d["topk_w"], k, H,
                        expert_norm=True, resid=d["resid"], gain=d["gain"])
    dt = time.perf_counter() - t0
    return {"value": round(ntok / dt, 2), "unit": "tokens/s", "cores": 1,
            "sample": "%d tokens, per-expert norm + residual + next pre-norm (fp64 oracle)" % ntok}


if __name__ == "__main__":
    main()
